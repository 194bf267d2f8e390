// Batched decode (B >= 2 tokens): the union of the tokens' active lists is
// loaded once and multiplied on the matrix cores (PowerInfer reading report,
// Part A section 4.4: the gain falls as the batch grows because the tokens'
// active sets overlap less than fully; the union is what must be read).
//
//   k_union_bits                   per-token bitmaps of the lists
//   k_union_compact                ascending union list U and |U|
//   k_union_up      (MFMA)         A[u][t] = W_up[U_u].x_t (+ gate), bias,
//                                  activation, zeroed where t did not select U_u
//   k_union_down    (MFMA)         Y[t] = sum_u A[u][t] * W_down[U_u, :]
//
// Each token's result equals its single-token result up to rounding: a
// neuron outside a token's own list contributes exactly 0 to that token.  A
// is stored in fp16 for the matrix-core down product (each activation
// rounded once, a relative error of at most 2^-11 per term, so about 3e-4 in
// y's relative L2 norm); the weights are fp16 already and the sums fp32.
#include "common.hpp"
#include "internal.hpp"
#include "ring.hpp"

namespace pi {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// ---------------------------------------------------------------------------
// Per-token bitmaps of the lists: tokbits[t][w] bit k = token t selected
// neuron 32w + k.  Every word is written, so no clearing pass is needed: the
// lists are strictly ascending, so the entries of one word form a run; the
// run's first entry ORs the run's bits (a segmented OR over the wave, then
// the entries past the wave's end, at most 31, loaded with the wave's own
// entries) and writes the word, and also
// zeroes the words strictly between the previous entry's word and its own;
// the words before the first entry's word and after the last one's are
// zeroed grid-wide.  Workgroups of token 0 also zero the compaction's count
// slots, its error word and the arrival counters of the up GEMM's row blocks.
__global__ __launch_bounds__(256) void k_union_bits(const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ count, int ffn, int nw,
                                                    uint32_t* __restrict__ tokbits, uint64_t* __restrict__ slots,
                                                    int nslots, uint32_t* __restrict__ upctr, int nup,
                                                    uint32_t* __restrict__ uerr) {
    const int t = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    const int stride = gridDim.x * 256;
    if (t == 0) {
        for (int i = blockIdx.x * 256 + tid; i < nup; i += stride) upctr[i] = 0u;
        for (int i = blockIdx.x * 256 + tid; i < nslots; i += stride) slots[i] = 0ull;
        if (blockIdx.x == 0 && tid == 0) *uerr = 0u;
    }
    const int cnt = clampi(count[t], 0, ffn);
    const int32_t* lst = idx + (size_t)t * ffn;
    uint32_t* out = tokbits + (size_t)t * nw;
    // ids are read clamped to [0, ffn): a list that breaks the contract gives
    // wrong bits but no access outside the bitmaps (PI_CHECK_IDX reports it)
    for (int j0 = blockIdx.x * 256 + (tid & ~63); j0 < cnt; j0 += stride) {   // whole waves
        // one round of loads: the wave's 64 entries, the 32 after them (a word
        // holds at most 32 entries, so the run at the wave's end ends there)
        // and, in lane 0, the entry before the wave
        const int j = j0 + lane, ja = j0 + 64 + lane;
        const bool in = j < cnt, ina = lane < 32 && ja < cnt;
        const int i = in ? clampi(lst[j], 0, ffn - 1) : 0;
        const int ia = ina ? clampi(lst[ja], 0, ffn - 1) : 0;
        const int ip = lane == 0 && j0 > 0 ? clampi(lst[j0 - 1], 0, ffn - 1) : 0;
        const int w = in ? (i >> 5) : -1 - lane;   // lanes past the list match no one
        uint32_t bits = in ? (1u << (i & 31)) : 0u;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {   // OR of this lane's entry and the rest of its run in the wave
            const uint32_t ob = __shfl_down(bits, off, 64);
            const int ow = __shfl_down(w, off, 64);
            if (lane + off < 64 && ow == w) bits |= ob;
        }
        const int wup = __shfl_up(w, 1, 64);
        const int w63 = __shfl(w, 63, 64);
        // the bits of the run that goes on past the wave: the entries after
        // it in word w63
        uint32_t xb = ina && (ia >> 5) == w63 ? 1u << (ia & 31) : 0u;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) xb |= __shfl_xor(xb, off, 64);
        if (!in) continue;
        const int wprev = j == 0 ? -1 : (lane == 0 ? ip >> 5 : wup);
        if (wprev == w) continue;   // not the first entry of its word
        if (w63 == w) bits |= xb;
        out[w] = bits;
        for (int g = j == 0 ? w : wprev + 1; g < w; ++g) out[g] = 0u;   // (the first entry: none)
    }
    // the words before the first entry's word and after the last one's
    const int wfirst = cnt > 0 ? clampi(lst[0], 0, ffn - 1) >> 5 : nw;
    const int wlast = cnt > 0 ? clampi(lst[cnt - 1], 0, ffn - 1) >> 5 : -1;
    for (int w = blockIdx.x * 256 + tid; w < nw; w += stride)
        if (w < wfirst || w > wlast) out[w] = 0u;
}

// Union compaction in one pass.  Workgroup g of G (at most kCompactWG, all
// resident at once) owns a contiguous range of 64-neuron tiles; each wave ORs
// the tokens' words of its tiles (lane l takes token l) into the tiles'
// union bitmaps, kept in LDS.  The workgroup publishes its count as one
// tagged 64-bit word {1, count} (the slots are zeroed by k_union_bits), sums
// the counts of workgroups 0..g-1 as they appear (a bounded wait: every
// workgroup publishes before it waits, so the wait ends), and writes its own
// entries of the ascending union list in parallel, each lane its neuron at
// its rank.  The last workgroup writes |U|.  A wait that overruns counts the
// missing workgroup as empty and marks its slot: the list is then short but
// stays in bounds, |U| is written as 0 and the error word is set, which
// k_union_reduce answers with NaN in every token's y.
constexpr int kCompactWG = 256;
// Grids shaped to fill whole waves assume the 256 CUs of an MI355X (on
// another device they are only less well shaped).
constexpr int kDeviceCUs = 256;
constexpr int kCompactTiles = 1024;   // tiles per workgroup held in LDS
constexpr int kCompactWait = 1 << 16;

__global__ __launch_bounds__(256) void k_union_compact(const uint32_t* __restrict__ tokbits, int ffn, int nw, int B,
                                                       uint64_t* __restrict__ slots,
                                                       int32_t* __restrict__ ulist,
                                                       uint32_t* __restrict__ ucount,
                                                       uint32_t* __restrict__ uerr) {
    __shared__ uint64_t s_m[kCompactTiles];
    __shared__ uint32_t s_wcnt[4];
    __shared__ uint32_t s_base, s_err;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ntiles = (ffn + 63) / 64;
    const int G = gridDim.x, g = blockIdx.x;
    const int t0 = (int)((long long)ntiles * g / G), t1 = (int)((long long)ntiles * (g + 1) / G);
    const int tw = (t1 - t0 + 3) / 4;   // tiles per wave
    uint32_t cnt = 0;
    for (int k = 0; k < tw; ++k) {
        const int tl = wave * tw + k, tile = t0 + tl;
        if (tile >= t1) break;
        // two tokens a lane, their four words loaded together; tokens past B
        // read token B - 1 again (the OR is unchanged) and a high word past
        // the bitmap reads the low one (dropped)
        const int wl = 2 * tile, wh = min(2 * tile + 1, nw - 1);
        const bool hv = 2 * tile + 1 < nw;
        uint64_t m = 0;
        for (int tb0 = 0; tb0 < B; tb0 += 128) {
            const size_t ra = (size_t)min(tb0 + lane, B - 1) * nw, rb = (size_t)min(tb0 + 64 + lane, B - 1) * nw;
            const uint32_t la = tokbits[ra + wl], ha = tokbits[ra + wh];
            const uint32_t lb = tokbits[rb + wl], hb = tokbits[rb + wh];
            m |= (uint64_t)(la | lb) | ((uint64_t)(hv ? ha | hb : 0u) << 32);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m |= __shfl_xor(m, off, 64);
        if (lane == 0) s_m[tl] = m;
        cnt += (uint32_t)__popcll(m);
    }
    if (lane == 0) s_wcnt[wave] = cnt;
    if (tid == 0) s_err = 0u;
    __syncthreads();
    const uint32_t total = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
    if (tid == 0) __hip_atomic_store(&slots[g], (1ull << 32) | total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wave == 0) {
        uint32_t sum = 0, err = 0;
        for (int j0 = 0; j0 < g; j0 += 64) {
            const int j = j0 + lane;
            if (j < g) {
                uint64_t v = __hip_atomic_load(&slots[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int n = 0; (v >> 32) == 0u; ++n) {
                    if (n == kCompactWait) {
                        v = 2ull << 32;   // give up: counted as empty, marked as an error
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                    v = __hip_atomic_load(&slots[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
                sum += (uint32_t)v;
                err |= (uint32_t)(v >> 32) & 2u;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            sum += __shfl_xor(sum, off, 64);
            err |= __shfl_xor(err, off, 64);
        }
        if (lane == 0) {
            s_base = sum;
            s_err = err;
        }
    }
    __syncthreads();
    uint32_t pos = s_base;
    for (int w2 = 0; w2 < wave; ++w2) pos += s_wcnt[w2];
    for (int k = 0; k < tw; ++k) {
        const int tl = wave * tw + k, tile = t0 + tl;
        if (tile >= t1) break;
        const uint64_t m = s_m[tl];
        if ((m >> lane) & 1ull) ulist[pos + rank_below(m)] = tile * 64 + lane;
        pos += (uint32_t)__popcll(m);
    }
    if (g == G - 1 && tid == 0) *ucount = s_err ? 0u : s_base + total;
    if (s_err && tid == 0) {
        __hip_atomic_store(&slots[g], (3ull << 32) | total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        st_flag(uerr, 1u);   // any workgroup's overrun: every token's y becomes NaN
    }
}

// ---------------------------------------------------------------------------
// Skinny GEMMs of the batched path (rows x tokens on the matrix cores, see
// ring.hpp), by XG = 8-token groups loaded: a ring of three stages of
// 512-byte row segments, or 256 or 128 where three stages of the larger ones
// would not fit in LDS.
constexpr int ring_seg(int nm, int nx, int xg, int rbw) {
    return 3 * (nm * 4 * rbw + nx * xg) * 4 <= 156 ? 4 : (3 * (nm * 4 * rbw + nx * xg) * 2 <= 156 ? 2 : 1);
}
// (the hidden layer at 128 tokens: 64-row blocks in four one-segment stages;
// its few rows make every row block split over many workgroups, and smaller
// blocks halve the pieces each workgroup writes)
template <int XG>
using HidCfg = RingCfg<1, 1, XG, rbw_hidden(XG), XG >= 16 ? 1 : ring_seg(1, 1, XG, rbw_hidden(XG)), XG >= 16 ? 4 : 3>;
template <int XG> using LogCfg = RingCfg<1, 2, XG, rbw_logits(XG), ring_seg(1, 2, XG, rbw_logits(XG)), 3>;
template <bool REGLU, int XG>
using UpCfg = RingCfg<REGLU ? 2 : 1, 1, XG, rbw_up(XG), ring_seg(REGLU ? 2 : 1, 1, XG, rbw_up(XG)), 3>;

// Up GEMM over the union rows: A[u][t] = W_up[U_u] . x_t (+ the gate
// product for ReGLU), then bias, activation and the token mask (zero where
// token t did not select neuron U_u), stored token-major in fp16: aT[t][u],
// for every token slot t < Bp (zero past B) and for u up to the next multiple
// of 8 past |U| (zero past |U|).
template <int KIND>
struct UpEpi {
    const int32_t* ulist;
    const float* bup;
    const float* bg;
    const uint32_t* tokbits;
    int nw, B, Bp, lda, U, U8;
    h16* a;
    struct Row {
        int nrow;
        float bu, bgv;
    };
    // (the ring runs no epilogue when |U| = 0, so U - 1 is a valid entry;
    // loads are unconditional at clamped addresses and their values masked
    // afterwards: loads under a branch make the compiler wait for all
    // outstanding memory operations, the previous outputs' stores included)
    __device__ Row row(int uu) const {
        const bool ok = uu < U;
        const int nrow = settle(ulist[min(uu, U - 1)]);
        const float bu = settle(bup ? bup[nrow] : 0.f);
        const float bgv = settle((KIND != 0 && bg) ? bg[nrow] : 0.f);
        return Row{ok ? nrow : 0, ok ? bu : 0.f, ok ? bgv : 0.f};
    }
    // (no early exit: every use of the row's loads sits on the path all
    // threads take, so the compiler waits for them once)
    template <int E>
    __device__ void apply(int uu, const Row& r, const int (&t)[E], const float (&vu)[E], const float (&vg)[E]) const {
        uint32_t bits[E];
#pragma unroll
        for (int k = 0; k < E; ++k)   // the E mask words in flight together
            bits[k] = tokbits[(size_t)min(t[k], B - 1) * nw + (r.nrow >> 5)];
#pragma unroll
        for (int k = 0; k < E; ++k) bits[k] = settle(bits[k]);
        float av[E];
#pragma unroll
        for (int k = 0; k < E; ++k) {
            // zero past |U| (the down GEMM reads whole 8-entry chunks) and
            // for the tokens that did not select the neuron
            const bool on = uu < U && t[k] < B && ((bits[k] >> (r.nrow & 31)) & 1u);
            av[k] = on ? ffn_act<KIND>(vu[k] + r.bu, KIND != 0 ? vg[k] + r.bgv : 0.f) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const h16 h = (h16)av[k];
            if (t[k] < Bp && uu < U8) a[(size_t)t[k] * lda + uu] = h;
        }
    }
};

template <class C, int KIND>
__global__ __launch_bounds__(256) void k_union_up(RingArgs a, const uint32_t* __restrict__ ucount, int ffn,
                                                  const float* __restrict__ bup, const float* __restrict__ bg,
                                                  const uint32_t* __restrict__ tokbits, int nw, int Bp, int lda,
                                                  h16* __restrict__ aT) {
    __shared__ __align__(16) char lds[C::LDS];
    const int U = (int)min(*ucount, (uint32_t)ffn);
    const UpEpi<KIND> epi{a.rowlist, bup, bg, tokbits, nw, a.B, Bp, lda, U, min((U + 7) & ~7, lda), aT};
    ring_gemm<C, true, true>(a, U, lds, epi);
}

// ---------------------------------------------------------------------------
// Batched predictor.  Hidden layer: H = act(P1 X^T + b1), written token-major
// as an fp16 hi/lo pair (h itself is never rounded to fp16: hi + lo carries
// about 22 significant bits).  P1 has few rows and long ones, so every row
// block is split over many workgroups and k_bpred_hidden_finish adds the
// pieces.  Workgroup 0 also zeroes the logits kernel's row-block counters,
// which that kernel (next but one on the stream) expects at 0.
struct HiddenEpi {
    const float* b1;
    int relu, r, B, ldh;
    h16* h_hi;
    h16* h_lo;
    struct Row {
        float b;
    };
    __device__ Row row(int j) const { return Row{settle(b1 ? b1[min(j, r - 1)] : 0.f)}; }
    // the value first, the store under the condition (see UpEpi)
    __device__ void store(int j, int t, float v, float b) const {
        const float sv = v + b;
        const float hv = relu ? fmaxf(sv, 0.f) : sv;
        const h16 hi = (h16)hv;
        const h16 lo = (h16)(hv - (float)hi);
        if (j < r && t < B) {
            h_hi[(size_t)t * ldh + j] = hi;
            h_lo[(size_t)t * ldh + j] = lo;
        }
    }
    template <int E>
    __device__ void apply(int j, const Row& rw, const int (&t)[E], const float (&v)[E], const float (&)[E]) const {
#pragma unroll
        for (int k = 0; k < E; ++k) store(j, t[k], v[k], rw.b);
    }
    __device__ void operator()(int j, int t, float v, float) const { store(j, t, v, row(j).b); }
};

template <class C>
__global__ __launch_bounds__(256) void k_bpred_hidden(RingArgs a, HiddenEpi epi, uint32_t* __restrict__ lctr,
                                                      int nlctr) {
    __shared__ __align__(16) char lds[C::LDS];
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < nlctr; i += 256) lctr[i] = 0u;
    ring_gemm<C, false, false>(a, a.nrows, lds, epi);
}

template <class C>
__global__ __launch_bounds__(256) void k_bpred_hidden_finish(RingArgs a, HiddenEpi epi, int G0) {
    ring_finish<C>(a, a.nrows, G0, epi);
}

// Hidden layer for groups of at most 8 tokens, on the vector units: one wave
// per P1 row streams the whole row once and takes the TB dot products against
// the group's x, staged in LDS by direct-to-LDS loads that go out behind the
// row's loads (tokens past B repeat token B - 1; their sums are dropped).  It
// writes h straight into the hi/lo pair the logits GEMM reads, so no K-split
// pieces and no finishing kernel.  Workgroup 0 zeroes the logits counters.
// x takes TB x roundup(d/8, 64) x 16 bytes of LDS: kHidValuChunks bounds d.
constexpr int hid_valu_chunks(int TB) { return TB <= 4 ? 2048 : 1152; }   // d <= 16384 / 9216
template <int TB>
__global__ __launch_bounds__(256) void k_bpred_hidden_valu(const h16* __restrict__ x, int B, int d,
                                                           const h16* __restrict__ P1, HiddenEpi epi,
                                                           uint32_t* __restrict__ lctr, int nlctr) {
    __shared__ __align__(16) u32x4 sx[TB * hid_valu_chunks(TB)];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (blockIdx.x == 0)
        for (int i = tid; i < nlctr; i += 256) lctr[i] = 0u;
    const int r = epi.r;
    const int row = blockIdx.x * 4 + wave;
    const h16* prow = P1 + (size_t)min(row, r - 1) * d;
    const int nch = d >> 3;
    const int ncp = (nch + 63) & ~63;   // LDS chunks per token
    u32x4 w[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) w[u] = ld16_stream(prow + (size_t)min(lane + u * 64, nch - 1) * 8);
    // x behind the row: block b = (token, 64 chunks) -> LDS [token][chunk]
    const uint32_t sbase = lds_addr(sx);
    const int nbt = ncp / 64;
    for (int b = wave; b < TB * nbt; b += 4) {
        const int t = b / nbt, c0 = (b % nbt) * 64;
        dma16(x + (size_t)min(t, B - 1) * d + (size_t)min(c0 + lane, nch - 1) * 8,
              sbase + (uint32_t)(t * ncp + c0) * 16u);
    }
    wait_vm<0>();
    ring_barrier();
    float acc[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[t] = 0.f;
    for (int c0 = lane; c0 < nch; c0 += 64 * 16) {
        if (c0 != lane) {   // rows longer than 8192: the next 16 chunks per lane
#pragma unroll
            for (int u = 0; u < 16; ++u) w[u] = ld16_stream(prow + (size_t)min(c0 + u * 64, nch - 1) * 8);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int c = c0 + u * 64;
            if (c < nch) {
#pragma unroll
                for (int t = 0; t < TB; ++t) acc[t] = dot8_h(w[u], sx[t * ncp + c], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) {
        const float v = group_sum<64>(acc[t]);
        if (lane == t && row < r) epi(row, t, v, 0.f);   // drops t >= B
    }
}

// Logits: Z = P2 H^T + b2 with both halves of h, then the strict test
// z > thr per (neuron, token); every 32 neurons give one 32-bit mask word per
// token (bit k = neuron 32*word + k).  Each half of a wave holds 32 neurons
// of one token: one ballot gives two words.
// The rows are neurons hot .. ffn - 1 (a.W[0] starts at P2 row hot, a.nrows =
// ffn - hot; hot is a multiple of 32, so each half-wave's 32 rows are still
// one mask word).  The words of the hot prefix are the compaction's.
struct LogitsEpi {
    const float* b2;
    float thr;
    uint32_t* masks32;
    int nw, hot, nr, B;
    struct Row {
        float b;
    };
    __device__ Row row(int i) const { return Row{settle(b2 ? b2[hot + min(i, nr - 1)] : 0.f)}; }
    template <int E>
    __device__ void apply(int i, const Row& rw, const int (&t)[E], const float (&v)[E], const float (&)[E]) const {
        const int n = hot + i, lane = threadIdx.x & 63;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const float z = v[k] + rw.b;
            const bool on = (i < nr) & (t[k] < B) & (z > thr);
            const uint64_t m = __ballot(on);
            if ((lane & 31) == 0 && i < nr && t[k] < B)
                masks32[(size_t)t[k] * nw + (n >> 5)] = (uint32_t)(m >> (lane & 32));
        }
    }
};

template <class C>
__global__ __launch_bounds__(256) void k_bpred_logits(RingArgs a, const float* __restrict__ b2, float thr,
                                                      uint32_t* __restrict__ masks32, int ffn, int hot) {
    __shared__ __align__(16) char lds[C::LDS];
    static_assert(C::RB % 32 == 0, "a half-wave must hold 32 neurons of one token");
    const LogitsEpi epi{b2, thr, masks32, (ffn + 31) / 32, hot, a.nrows, a.B};
    ring_gemm<C, false, true>(a, a.nrows, lds, epi);
}

// Logits for more than 32 tokens with h held in registers.  Workgroup
// (q, range) takes the 32 tokens of group q and a range of 32-row blocks of
// P2 (rows hot ..); wave w keeps both halves of h for eighths w and w + 4 of
// K (r / 4 entries: KS = r / 64 MFMA steps, 8 registers a step), so that
// only P2 goes through LDS.  A stage is one half of K of a 32-row block
// (32 x r / 2 halves, by direct-to-LDS loads in the blocks of ring.hpp: 8
// rows x 128 bytes per load, slots swizzled by row); in each half every
// wave multiplies its eighth, and the ring of four stages keeps three in
// flight.  After the second half of a block the four waves' partial sums go
// through LDS, are added in wave order, and give the mask words as in
// k_bpred_logits.  No row is split across workgroups, and h is read once per
// workgroup instead of once per row block.  The token groups of one row
// range are 8 workgroup indices apart: on one XCD, and dispatched together,
// so that three of the four reads of a P2 row hit its L2.
constexpr int kTqMaxR = 1024;                 // h registers: r / 64 <= 16 steps
constexpr int kTqRedE = 65, kTqRedW = 1040;   // partial sums: [wave][16 elements][65 floats]
constexpr int kTqStages = 4;
constexpr int kTqMaxBlocks = 64;              // 32-row blocks per workgroup (their biases sit in LDS)
inline int logits_tq_ranges(int B) {
    const int nq = (B + 31) / 32;
    const int rr8 = kDeviceCUs / (8 * nq);
    return 8 * (rr8 > 0 ? rr8 : 1);
}
// r = 256, 512 or 1024 (KS = r / 64, a compile-time count so that a wave's
// LDS reads all go out ahead of its MFMAs), at most kTqMaxBlocks row blocks
// per workgroup
inline bool logits_tq_fits(int B, int r, int nr) {
    const long long nrb = (nr + 31) / 32, nrg = logits_tq_ranges(B);
    return B > 32 && (r == 256 || r == 512 || r == 1024) && (nrb + nrg - 1) / nrg <= kTqMaxBlocks;
}

__device__ __forceinline__ void wait_lds_ops() {   // lgkmcnt(0) only (vector memory not waited on)
    __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x3 << 14));
}

template <int KS>
__global__ __launch_bounds__(256) void k_bpred_logits_tq(const h16* __restrict__ P2, int nr, int hot,
                                                         const h16* __restrict__ h_hi,
                                                         const h16* __restrict__ h_lo, int ldh, int B,
                                                         int nq, int nranges, const float* __restrict__ b2,
                                                         float thr, uint32_t* __restrict__ masks32, int ffn) {
    constexpr int r = KS * 64;
    constexpr int HB = KS / 2;            // 8-chunk blocks per row group in a half-K stage
    constexpr int IPW = HB;               // loads per wave per stage (4 row groups x HB blocks)
    constexpr int STG = 32 * (r / 2) * 2; // bytes per stage
    __shared__ __align__(16) char lds[kTqStages * 32 * (kTqMaxR / 2) * 2];
    __shared__ float red[4 * kTqRedW];
    __shared__ float s_b2[kTqMaxBlocks * 32];
    static_assert(IPW * (kTqStages - 2) < 64, "loads in flight");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, kh = lane >> 5;
    // workgroup b: XCD slot b % 8, then token group, then range group
    const int b = blockIdx.x, hi8 = b >> 3;
    const int q = hi8 % nq, rg = (b & 7) + 8 * (hi8 / nq);
    const int nrb = (nr + 31) / 32;
    const int rb0 = (int)((long long)rg * nrb / nranges), rb1 = (int)((long long)(rg + 1) * nrb / nranges);
    const int ns = 2 * (rb1 - rb0);       // stages: two halves of K per row block
    if (ns <= 0) return;
    const h16* W = P2 + (size_t)hot * r;
    const uint32_t lbase = lds_addr(lds);

    // this wave's h: token q*32 + li; step k < KS/2 of half f is chunk
    // f*(r/16) + w*(r/64) + 2k + kh, in register f*(KS/2) + k (slots past B
    // read the buffer's padding)
    f16x8 hh[KS], hl[KS];
    {
        const size_t tro = (size_t)(q * 32 + li) * ldh + (size_t)(wave * (r >> 6) + kh) * 8;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int k = 0; k < KS / 2; ++k) {
                hh[f * (KS / 2) + k] = *reinterpret_cast<const f16x8*>(h_hi + tro + f * (r / 2) + k * 16);
                hl[f * (KS / 2) + k] = *reinterpret_cast<const f16x8*>(h_lo + tro + f * (r / 2) + k * 16);
            }
    }
    // the range's biases to LDS, and h settled, before any stage goes out: a
    // compiler wait for a load inside the stage loop would drain the ring
    for (int i = tid; i < (ns / 2) * 32; i += 256) s_b2[i] = b2 ? b2[hot + min(rb0 * 32 + i, nr - 1)] : 0.f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        hh[k] = settle(hh[k]);
        hl[k] = settle(hl[k]);
    }
    __syncthreads();
    auto issue1 = [&](int st, int i) {
        const uint32_t dst = lbase + (uint32_t)((st % kTqStages) * STG);
        const int rb = rb0 + (st >> 1), half = st & 1;
        const int blk = wave + 4 * i;
        const int g = blk / HB, cg = blk % HB;
        const int rr = g * 8 + (lane >> 3);   // the lane's row within the block of 32
        const int row = min(rb * 32 + rr, nr - 1);
        const int chunk = half * (r / 16) + cg * 8 + ((lane & 7) ^ blk_swz(rr));
        dma16(W + (size_t)row * r + chunk * 8, dst + (uint32_t)blk * 1024u);
    };
    auto issue = [&](int st) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) issue1(st, i);
    };
    const int nw = (ffn + 31) / 32;
#pragma unroll
    for (int j = 0; j < kTqStages - 1; ++j)
        if (j < ns) issue(j);
    // one half of K of row block rb (stage s): every wave multiplies its
    // eighth.  The LDS reads go out first; the next stage's loads go out
    // between the MFMAs, one per two (as in ring.hpp)
    auto half_stage_m = [&](int s, auto HALF, ring_f32x16& acc, auto MORE) {
        constexpr int F = decltype(HALF)::value;
        if (s + kTqStages - 2 < ns) wait_vm<(kTqStages - 2) * IPW>();   // stage s is in
        else wait_vm<0>();
        ring_barrier();   // every wave's loads of stage s are in; everyone is past stage s - 1 and the sums
        const char* buf = lds + (s % kTqStages) * STG;
        const int g = li >> 3;
        f16x8 a[KS / 2];
#pragma unroll
        for (int k = 0; k < KS / 2; ++k) {
            const int c = wave * (r >> 6) + 2 * k + kh;   // chunk within the half
            a[k] = *reinterpret_cast<const f16x8*>(buf + (g * HB + (c >> 3)) * 1024 + blk_off(li, c & 7));
        }
        __builtin_amdgcn_sched_barrier(0);
        static_assert(KS / 2 == IPW, "one load per two MFMAs");
#pragma unroll
        for (int k = 0; k < KS / 2; ++k) {
            if constexpr (decltype(MORE)::value) issue1(s + kTqStages - 1, k);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[k], hh[F * (KS / 2) + k], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[k], hl[F * (KS / 2) + k], acc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // (a separate copy for the last stages, which load nothing: a load under
    // a branch inside the MFMA sequence would be gathered into one block)
    auto half_stage = [&](int s, auto HALF, ring_f32x16& acc) {
        if (s + kTqStages - 1 < ns) half_stage_m(s, HALF, acc, std::true_type{});
        else half_stage_m(s, HALF, acc, std::false_type{});
    };
    for (int rb = rb0; rb < rb1; ++rb) {
        const int s = 2 * (rb - rb0);
        ring_f32x16 acc = {};
        half_stage(s, std::integral_constant<int, 0>{}, acc);
        half_stage(s + 1, std::integral_constant<int, 1>{}, acc);
        // element e of lane l: row (e/4)*8 + 4*(l/32) + e%4, token l%32
#pragma unroll
        for (int e = 0; e < 16; ++e) red[wave * kTqRedW + e * kTqRedE + lane] = acc[e];
        wait_lds_ops();
        ring_barrier();
        // wave w: tokens 4w + k (lanes 0-31) and 4w + k + 16 (lanes 32-63), row li
        const int e = ((li >> 3) << 2) + (li & 3), hb = ((li >> 2) & 1) << 5;
        const int grow = rb * 32 + li;
        const float brow = s_b2[(rb - rb0) * 32 + li];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int n = 4 * wave + k + (kh << 4), t = q * 32 + n;
            float v = 0.f;
#pragma unroll
            for (int p = 0; p < 4; ++p) v += red[p * kTqRedW + e * kTqRedE + hb + n];
            const bool on = (grow < nr) & (t < B) & (v + brow > thr);
            const uint64_t m = __ballot(on);
            if (li == 0 && t < B) masks32[(size_t)t * nw + ((hot + rb * 32) >> 5)] = (uint32_t)(m >> (lane & 32));
        }
    }
}

// One workgroup per token: the token's 32-bit tile masks in neuron order ->
// popcount prefix -> ascending idx and count.  Thread k takes words 2k and
// 2k + 1 of each quarter of a 2048-word round (one block-wide scan per
// quarter), so the dense words of a hot-first layer spread over many threads
// while each thread writes in four loops.  The first hotw words
// (the always-listed hot prefix) count as all ones and are not read.
__global__ __launch_bounds__(256) void k_bpred_compact(const uint32_t* __restrict__ masks32, int ffn, int hotw,
                                                       int32_t* __restrict__ idx, int32_t* __restrict__ count) {
    __shared__ uint32_t s_part[16];
    const int tok = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ntiles = (ffn + 31) / 32;
    const uint32_t* mk = masks32 + (size_t)tok * ntiles;
    int32_t* out = idx + (size_t)tok * ffn;
    uint32_t base = 0;
    for (int t0 = 0; t0 < ntiles; t0 += 2048) {
        uint32_t m8[8], c4[4], i4[4];
#pragma unroll
        for (int q = 0; q < 8; ++q) {   // words 2k, 2k + 1 of quarter q / 2
            const int t = t0 + (q >> 1) * 512 + tid * 2 + (q & 1);
            m8[q] = t < hotw ? 0xFFFFFFFFu : (t < ntiles ? mk[t] : 0u);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            c4[h] = (uint32_t)(__popc(m8[2 * h]) + __popc(m8[2 * h + 1]));
            uint32_t incl = c4[h];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t v = __shfl_up(incl, off, 64);
                if (lane >= off) incl += v;
            }
            i4[h] = incl;
            if (lane == 63) s_part[h * 4 + wave] = incl;
        }
        __syncthreads();
        uint32_t run = base;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t pos = run + i4[h] - c4[h];
            for (int w2 = 0; w2 < wave; ++w2) pos += s_part[h * 4 + w2];
            run += s_part[h * 4] + s_part[h * 4 + 1] + s_part[h * 4 + 2] + s_part[h * 4 + 3];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                uint32_t m = m8[2 * h + e];
                const int t = t0 + h * 512 + tid * 2 + e;
                while (m) {
                    out[pos++] = t * 32 + __builtin_ctz(m);
                    m &= m - 1;
                }
            }
        }
        base = run;
        __syncthreads();
    }
    if (tid == 0) count[tok] = (int32_t)base;
}

// ---------------------------------------------------------------------------
// Down GEMM.  Y[t][c] = sum_u A[t][u] W_down[U_u][c]: the contraction runs
// over union entries, i.e. across rows of W_down.  Grid = (128-column tiles,
// G chunks of the union list); a workgroup streams its chunk's rows of its
// column tile through an LDS ring, stages of KR union entries: 8-row x
// 128-byte blocks of W_down (by direct-to-LDS loads as in ring.hpp, with the
// slot swizzle dn_wswz; row ids taken from the chunk's list staged in LDS)
// and the stage's activations, hi and lo (see DownCfg).
//
// The matrix cores need K (union entries) along each lane's operand, while
// W_down holds columns along a row: ds_read_b64_tr_b16 transposes on the LDS
// read.  Within each 16-lane group, lane l gets element l % 4 of the 64-bit
// words read by lanes l/4, 4 + l/4, 8 + l/4 and 12 + l/4 (measured on
// gfx950); so when lane 4k + m reads row k, columns 4m .. 4m+3 of a 16-column
// group, lane j receives column j of rows 0..3.  Two such reads give a lane
// column l % 32 of the 8 union entries of its half (l / 32) of a 16-entry
// step, the A operand of v_mfma_f32_32x32x16_f16 (columns x entries); the B
// operand is 16 bytes of A[t][.] per lane.  Wave w owns columns 32w..32w+31
// of the tile for every token.  Chunk partials go to the workspace and
// k_union_reduce adds them in chunk order (a kernel of its own: the sums of
// a tile's chunks spread over the whole device instead of one workgroup).
constexpr int kDnIds = 4096;   // union ids staged in LDS at a time (a window of the chunk)

// Wave w owns CB blocks of 32 columns (the tile is 128 CB columns): with 128
// tokens, two blocks per wave halve the activation bytes per W_down byte.
// A stage is KR union entries: 64, or 32 with 128 tokens, where a 64-entry
// stage (64 KB) would leave room for only two in LDS and the ring would hold
// a single stage in flight; 32-entry stages give it four.  An activation
// block is what one wave-wide load moves, TPB tokens x KR entries, the lanes
// of one token on its contiguous bytes (so that the load unit merges them):
// 8 tokens x 128 bytes laid out as the blocks of ring.hpp, or 16 tokens x 64
// bytes, [token][slot], chunk c of token t in slot c ^ ((t / 4) % 4), which
// puts the 16 tokens of one LDS read phase on 16 different 4-bank groups.
template <int XG_>
struct DownCfg {
    static constexpr int XG = XG_;
    static constexpr int NB = (XG + 3) / 4, BP = 32 * NB;
    static constexpr int CB = XG >= 16 ? 2 : 1;
    static constexpr int CT = 128 * CB;                            // columns per tile
    static constexpr int KR = XG >= 16 ? 32 : 64;                  // union entries per stage
    static constexpr int TPB = 512 / KR;                           // tokens per activation block
    static constexpr int WBLK = (KR / 8) * (CT / 64);              // W_down blocks per stage
    static constexpr int ABA = (8 * XG + TPB - 1) / TPB;           // activation blocks per array
    static constexpr int ABLK = ABA;                               // activation blocks
    static constexpr int NBLK = ((WBLK + ABLK + 3) / 4) * 4;       // padded to whole waves
    static constexpr int IPW = NBLK / 4;
    static constexpr int STAGE = NBLK * 1024;
    // ring depth: four 32-entry stages, else three stages where they fit
    // (which keeps two workgroups per CU at up to 16 tokens), else two
    static constexpr int NS = KR == 32 && 4 * STAGE + kDnIds * 4 <= 156 * 1024
                                  ? 4 : (3 * STAGE + kDnIds * 4 <= 156 * 1024 ? 3 : 2);
    static_assert(WBLK % 4 == 0 && IPW * (NS - 2) < 64, "loads per stage");
    static_assert(TPB == 8 || TPB == 16, "activation block shapes");
    // LDS byte offset in activation block tg of chunk c (8 entries) of token t
    static __device__ __forceinline__ int aoff(int tg, int c, int t) {
        return TPB == 8 ? blk_off(tg * 8 + (t & 7), c) : ((t & 15) << 6) + ((c ^ ((t >> 2) & 3)) << 4);
    }
    // the chunk that lane `lane` of activation block tg loads (its slot is lane % (64 / TPB))
    static __device__ __forceinline__ int achunk(int tg, int lane) {
        return TPB == 8 ? (lane & 7) ^ blk_swz(tg * 8 + (lane >> 3)) : (lane & 3) ^ ((lane >> 4) & 3);
    }
};

// Resident down workgroups per CU, by their LDS (the registers allow more).
template <int X>
constexpr int down_per_cu() {
    return (160 * 1024) / (DownCfg<X>::NS * DownCfg<X>::STAGE + kDnIds * 4);
}
static_assert(down_per_cu<1>() == 2 && down_per_cu<2>() == 2 && down_per_cu<16>() == 1, "down occupancy");

// The down grid is (column tiles, G chunks of the union).  A partial wave
// costs as much as a full one, so G fills whole waves of the workgroup slots
// of the device: of 1 to 4 waves, the best use of the slots, the fewest
// waves on a near tie (fewer chunk partials to add).
int union_down_chunks(int B, int d) {
    const int xg = ring_xg(B);
    const int ct = xg == 16 ? DownCfg<16>::CT : (xg == 8 ? DownCfg<8>::CT : (xg == 4 ? DownCfg<4>::CT
                 : (xg == 2 ? DownCfg<2>::CT : DownCfg<1>::CT)));
    const int per = xg == 16 ? down_per_cu<16>() : (xg == 8 ? down_per_cu<8>() : (xg == 4 ? down_per_cu<4>()
                  : (xg == 2 ? down_per_cu<2>() : down_per_cu<1>())));
    const int tiles = (d + ct - 1) / ct, slots = kDeviceCUs * per;
    int best = 1;
    double use = -1.0;
    for (int k = 1; k <= 4; ++k) {
        const int g = std::min(64, std::max(1, k * slots / tiles));
        const int waves = (tiles * g + slots - 1) / slots;
        const double u = (double)tiles * g / ((double)waves * slots);
        if (u > use + 0.02) {
            use = u;
            best = g;
        }
    }
    return best;
}

// W_down blocks: 8 union entries x 128 bytes (64 columns), [entry][slot] as
// the blocks of ring.hpp, but chunk c of entry k in slot c ^ dn_wswz(k): the
// transposing reads below take entries 0-3 (or 4-7) at 4 column quads of two
// neighbouring chunks per 16 lanes, and entries k and k + 2 (the same half of
// the 256-byte bank cycle) must then fall in different 64-byte quarters.
__device__ __forceinline__ int dn_wswz(int k) { return (k & 2) << 1; }

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ f16x4 lds_read8_tr(const char* p) {
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_char*)p));
}

template <class C>
__global__ __launch_bounds__(256) void k_union_down(const h16* __restrict__ Wd, int d, int ffn,
                                                    const int32_t* __restrict__ ulist,
                                                    const uint32_t* __restrict__ ucount,
                                                    const h16* __restrict__ aT, int B, int Bp, int lda,
                                                    float* __restrict__ partial, int G,
                                                    const h16* __restrict__ zsrc) {
    __shared__ __align__(16) char lds[C::NS * C::STAGE];
    __shared__ int32_t s_ids[kDnIds];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 31, kh = lane >> 5;
    const int tile = blockIdx.x, chunk = blockIdx.y;
    const int U = (int)min(*ucount, (uint32_t)ffn);
    // chunk starts are multiples of 8: 16-byte activation loads stay aligned
    const int per = (((U + G - 1) / G) + 7) & ~7;
    const int u0 = min(U, chunk * per), u1 = min(U, u0 + per);
    const int n_ids = u1 - u0;
    const int n = (n_ids + C::KR - 1) / C::KR;
    const int c0 = tile * C::CT;
    // the chunk's union ids, kDnIds at a time (a window: kDnIds / KR stages)
    auto load_ids = [&](int w0) {
        const int nw = min(n_ids - w0, kDnIds);
        for (int i0 = 0; i0 < nw; i0 += 256 * 8) {   // 8 loads in flight per thread
            int v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = ulist[u0 + w0 + min(i0 + k * 256 + tid, max(nw - 1, 0))];
            // unconditional stores (i0 <= kDnIds - 2048 keeps them in the
            // window; slots past nw hold a repeated id that no stage uses):
            // a conditional store would leave loads pending across the branch
            // and the compiler would then drain every DMA before the MFMA reads
#pragma unroll
            for (int k = 0; k < 8; ++k) s_ids[i0 + k * 256 + tid] = v[k];
        }
    };
    static_assert(kDnIds % C::KR == 0, "whole stages per id window");
    static_assert(kDnIds % (256 * 8) == 0, "id window loads cover whole 2048-id rounds");
    int window = 0;
    load_ids(0);
    __syncthreads();
    const uint32_t lbase = (uint32_t)(size_t)(lds_void_ptr)lds;

    // this thread's loads: block b = wave + 4i; weight blocks first (WBLK is a
    // multiple of 4, so block i is a weight block exactly when i < WBLK / 4)
    int wofs[C::IPW];       // weight: row-in-stage; activation: token row offset
    int kofs[C::IPW];       // weight: column offset; activation: entry offset in the stage
    const h16* abase[C::IPW];
#pragma unroll
    for (int i = 0; i < C::IPW; ++i) {
        const int b = wave + 4 * i;
        if (i < C::WBLK / 4) {
            // lane j: entry 8 rg + j / 8 of the stage, slot j % 8 (see dn_wswz)
            const int rg = b / (C::CT / 64), cs = b % (C::CT / 64);
            wofs[i] = rg * 8 + (lane >> 3);
            kofs[i] = c0 + cs * 64 + (((lane & 7) ^ dn_wswz(lane >> 3)) << 3);
            abase[i] = nullptr;
        } else {
            // lane j writes LDS bytes 16j.. of the block: token j / (64 / TPB)
            // of it, slot j % (64 / TPB)
            const int bx = b - C::WBLK;
            const int tg = bx;
            const int t = tg * C::TPB + lane / (64 / C::TPB);
            const bool real = bx < C::ABLK && t < B;
            abase[i] = real ? aT + (size_t)t * lda : nullptr;
            wofs[i] = 0;
            kofs[i] = C::achunk(tg, lane) << 3;
        }
    }
    // stage st's sources: the union ids of its weight blocks from the window
    auto prep = [&](int st, const h16* (&p)[C::IPW]) {
        const int wst = st * C::KR / kDnIds;   // uniform: every wave issues the same stage
        if (wst != window) {
            // every wave has issued the previous window's last stage (it read
            // its ids then), so the window can be replaced; a rare stall
            __syncthreads();
            load_ids(wst * kDnIds);
            __syncthreads();
            window = wst;
        }
        int id[C::WBLK / 4];
#pragma unroll
        for (int i = 0; i < C::WBLK / 4; ++i)
            id[i] = clampi(s_ids[min(st * C::KR + wofs[i] - window * kDnIds, kDnIds - 1)], 0, ffn - 1);
#pragma unroll
        for (int i = 0; i < C::IPW; ++i) {
            if (i < C::WBLK / 4) {
                const bool ok = st * C::KR + wofs[i] < n_ids && kofs[i] < d;
                p[i] = ok ? Wd + (size_t)id[i] * d + kofs[i] : zsrc;
            } else {
                const int e = st * C::KR + kofs[i];
                p[i] = (abase[i] && e < n_ids) ? abase[i] + u0 + e : zsrc;
            }
        }
    };
    auto issue1 = [&](const h16* p, int q, int i) {
        const uint32_t dst = lbase + q * C::STAGE;
        if (i < C::WBLK / 4) dma16_stream(p, dst + (wave + 4 * i) * 1024);   // W_down: read once
        else dma16(p, dst + (wave + 4 * i) * 1024);
    };
    auto issue = [&](int st, int q) {
        const h16* p[C::IPW];
        prep(st, p);
#pragma unroll
        for (int i = 0; i < C::IPW; ++i) issue1(p[i], q, i);
    };

    f32x16 acc[C::CB][C::NB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) acc[cb][nb] = f32x16{};
    const int g = lane >> 4, j = lane & 15;

    wait_vm<0>();
#pragma unroll
    for (int jj = 0; jj < C::NS - 1; ++jj)
        if (jj < n) issue(jj, jj);
    // stage s; MORE: a stage s + NS - 1 exists.  All of the stage's LDS
    // reads go out first, then its MFMAs run back to back, with the next
    // stage's loads spread between them when there are at least two MFMAs
    // per load, else issued at once after the barrier (see ring.hpp)
    constexpr int NMF = C::KR / 16 * C::CB * C::NB;   // MFMAs per wave per stage
    constexpr bool kSpread = NMF >= 2 * C::IPW;
    auto stage = [&](int s, auto MORE) {
        if (s + C::NS - 2 < n) wait_vm<(C::NS - 2) * C::IPW>();
        else wait_vm<0>();
        ring_barrier();
        const int qn = (s + C::NS - 1) % C::NS;
        if constexpr (decltype(MORE)::value && !kSpread) issue(s + C::NS - 1, qn);
        const char* buf = lds + (s % C::NS) * C::STAGE;
        f16x4 w0[C::KR / 16][C::CB], w1[C::KR / 16][C::CB];
        f16x8 av[C::KR / 16][C::NB];
#pragma unroll
        for (int q = 0; q < C::KR / 16; ++q) {
            const int rg = 2 * q + kh;   // row group of this lane half's 8 entries
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) {
                // first of this lane's 4 columns in column block cb of the wave
                const int col = (wave * C::CB + cb) * 32 + 16 * (g & 1) + 4 * (j & 3);
                const int cs = col >> 6, ch = (col & 63) >> 3, quad = (col >> 2) & 1;
                const char* wb = buf + (rg * (C::CT / 64) + cs) * 1024 + quad * 8;
                const int k0 = j >> 2, k1 = k0 + 4;   // the block's rows this lane reads
                w0[q][cb] = lds_read8_tr(wb + (k0 << 7) + ((ch ^ dn_wswz(k0)) << 4));
                w1[q][cb] = lds_read8_tr(wb + (k1 << 7) + ((ch ^ dn_wswz(k1)) << 4));
            }
            const int c = 2 * q + kh;    // activation chunk (8 entries)
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                const int t = nb * 32 + li, tg = min(t / C::TPB, C::ABA - 1);
                av[q][nb] = *reinterpret_cast<const f16x8*>(buf + (C::WBLK + tg) * 1024 + C::aoff(tg, c, t));
            }
        }
        const h16* pn[C::IPW];
        if constexpr (decltype(MORE)::value && kSpread) prep(s + C::NS - 1, pn);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < C::KR / 16; ++q)
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb) {
                const f16x8 a8 = {w0[q][cb][0], w0[q][cb][1], w0[q][cb][2], w0[q][cb][3],
                                  w1[q][cb][0], w1[q][cb][1], w1[q][cb][2], w1[q][cb][3]};
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb) {
                    const int f = (q * C::CB + cb) * C::NB + nb;
                    if constexpr (decltype(MORE)::value && kSpread) {
#pragma unroll
                        for (int i = 0; i < C::IPW; ++i)
                            if (i * NMF / C::IPW == f) issue1(pn[i], qn, i);
                    }
                    acc[cb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a8, av[q][nb], acc[cb][nb], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
    };
    {
        int s = 0;
        for (; s + C::NS - 1 < n; ++s) stage(s, std::true_type{});
        for (; s < n; ++s) stage(s, std::false_type{});
    }
    // acc[cb][nb] element e of lane l: column (wave*CB + cb)*32 + 8*(e/4) + 4*(l/32) + e%4
    // of the tile, token nb*32 + l%32; four consecutive columns per 16-byte store
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
            const int t = nb * 32 + li;
            if (t >= B) continue;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int cc = c0 + (wave * C::CB + cb) * 32 + 8 * e4 + 4 * kh;
                if (cc < d) {
                    const f32x4 v = {acc[cb][nb][4 * e4], acc[cb][nb][4 * e4 + 1], acc[cb][nb][4 * e4 + 2],
                                     acc[cb][nb][4 * e4 + 3]};
                    *reinterpret_cast<f32x4*>(&partial[((size_t)chunk * Bp + t) * d + cc]) = v;
                }
            }
        }
}

// y[t][c] = sum over chunks g (in order) of partial[g][t][c]: four outputs
// (16 bytes) per thread, the G loads issued 8 at a time; 32-bit index
// arithmetic (B x d is far below 2^31; a 64-bit division per thread had made
// this kernel instruction-bound).  NaN for a token whose count is negative
// (the predictor's overrun report), and for every token when the union
// compaction overran its wait.  d is a multiple of 8 and y 16-byte aligned.
__global__ __launch_bounds__(256) void k_union_reduce(const float* __restrict__ partial, int B, int Bp,
                                                      int d, int G, float* __restrict__ y,
                                                      const int32_t* __restrict__ count,
                                                      const uint32_t* __restrict__ uerr) {
    const int dq = d >> 2;
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q >= B * dq) return;
    const int t = q / dq, c = (q - t * dq) * 4;
    f32x4* yo = reinterpret_cast<f32x4*>(y + (size_t)t * d + c);
    if (count[t] < 0 || *uerr != 0u) {
        const float nan = __builtin_nanf("");
        *yo = f32x4{nan, nan, nan, nan};
        return;
    }
    const float* p = partial + (size_t)t * d + c;
    const size_t gs = (size_t)Bp * d;   // one chunk's partials
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int g0 = 0; g0 < G; g0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            v[u] = g0 + u < G ? *reinterpret_cast<const f32x4*>(p + (size_t)(g0 + u) * gs) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            sum.x += v[u].x;
            sum.y += v[u].y;
            sum.z += v[u].z;
            sum.w += v[u].w;
        }
    }
    *yo = sum;
}

// PI_CHECK_IDX: one workgroup per token checks its list against the contract
// (count in [0, ffn], ids in [0, ffn), strictly ascending) after the FFN has
// run, and fills y_t with NaN if it breaks it.  The FFN kernels read ids
// clamped to [0, ffn), so a broken list never reads outside the weights.
__global__ __launch_bounds__(256) void k_check_idx(const int32_t* __restrict__ idx,
                                                   const int32_t* __restrict__ count, int ffn, int d,
                                                   float* __restrict__ y) {
    const int t = blockIdx.x, tid = threadIdx.x;
    const int c = count[t];
    const int32_t* lst = idx + (size_t)t * ffn;
    bool bad = c < 0 || c > ffn;
    const int n = bad ? 0 : c;
    for (int j = tid; j < n; j += 256) {
        const int i = lst[j];
        bad = bad || i < 0 || i >= ffn || (j > 0 && lst[j - 1] >= i);
    }
    if (!__syncthreads_or(bad)) return;
    const float nan = __builtin_nanf("");
    for (int k = tid; k < d; k += 256) y[(size_t)t * d + k] = nan;
}

hipError_t launch_check_idx(const int32_t* idx, const int32_t* count, int B, int ffn, int d, float* y,
                            hipStream_t s) {
    hipLaunchKernelGGL(k_check_idx, dim3(B), dim3(256), 0, s, idx, count, ffn, d, y);
    return hipGetLastError();
}

// Workgroups of a ring kernel that are resident on the device at once (at
// most kRingMaxWG, the size the piece areas are laid out for).
template <auto KERN>
static int ring_grid() {
    static const int g = [] {
        int dev = 0, cus = 0, per = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(KERN), 256, 0) != hipSuccess)
            return kRingMaxWG / 2;
        const int n = (per > 0 ? per : 1) * (cus > 0 ? cus : 1);
        return n < kRingMaxWG ? n : kRingMaxWG;
    }();
    return g;
}


hipError_t launch_union(int kind, const h16* x, int B, int d, int ffn, const h16* Wup,
                        const float* bup, const h16* Wg, const float* bg, const h16* Wd,
                        const int32_t* idx, const int32_t* count, float* y, const BatchLayout& L,
                        char* ws, char* hdr, hipStream_t s) {
    uint32_t* tokbits = reinterpret_cast<uint32_t*>(ws + L.tokbits);
    uint64_t* umasks = reinterpret_cast<uint64_t*>(ws + L.umasks);
    int32_t* ulist = reinterpret_cast<int32_t*>(ws + L.ulist);
    uint32_t* ucount = reinterpret_cast<uint32_t*>(ws + L.ucount);
    uint32_t* uerr = ucount + 1;   // the compaction's error word (the |U| slot is 256 bytes)
    h16* aT = reinterpret_cast<h16*>(ws + L.aT);
    float* partial = reinterpret_cast<float*>(ws + L.partial);
    uint32_t* upctr = reinterpret_cast<uint32_t*>(ws + L.upctr);
    const int nw = (ffn + 31) / 32;
    int gb = (ffn + 1023) / 1024;
    if (gb > 16) gb = 16;
    const int ntiles = (ffn + 63) / 64;
    int gc = (ntiles + 3) / 4;   // a tile per wave, up to kCompactWG workgroups
    if (gc > kCompactWG) gc = kCompactWG;
    hipLaunchKernelGGL(k_union_bits, dim3(gb, B), dim3(256), 0, s, idx, count, ffn, nw, tokbits, umasks, gc, upctr,
                       (ffn + kRingRows - 1) / kRingRows, uerr);
    hipLaunchKernelGGL(k_union_compact, dim3(gc), dim3(256), 0, s, tokbits, ffn, nw, B, umasks, ulist, ucount, uerr);
    RingArgs ra{};
    ra.W[0] = Wup;
    ra.W[1] = Wg;
    ra.ldw = d;
    ra.rowlist = ulist;
    ra.wrows = ffn;
    ra.nrows = 0;   // |U|, read on the device
    ra.X[0] = x;
    ra.ldx = d;
    ra.B = B;
    ra.K = d;
    ra.zsrc = reinterpret_cast<const h16*>(hdr + Sync::zero);
    ra.part = reinterpret_cast<float*>(ws + L.upart);
    ra.ctr = upctr;
#define PI_UP(K, N)                                                                                        \
    hipLaunchKernelGGL((k_union_up<UpCfg<(K != 0), N>, K>), dim3(ring_grid<k_union_up<UpCfg<(K != 0), N>, K>>()), \
                       dim3(256), \
                       0, s, ra, ucount, ffn, bup, bg, tokbits, nw, L.Bp, L.lda, aT)
#define PI_DN(X)                                                                                        \
    hipLaunchKernelGGL((k_union_down<DownCfg<X>>), dim3((d + DownCfg<X>::CT - 1) / DownCfg<X>::CT, L.G), dim3(256), \
                       0, s, Wd, d, ffn, ulist, ucount, \
                       aT, B, L.Bp, L.lda, partial, L.G, ra.zsrc)
    const int xg = ring_xg(B);
    if (kind == 2) {
        if (xg == 1) PI_UP(2, 1); else if (xg == 2) PI_UP(2, 2); else if (xg == 4) PI_UP(2, 4);
        else if (xg == 8) PI_UP(2, 8); else PI_UP(2, 16);
    } else if (kind == 1) {
        if (xg == 1) PI_UP(1, 1); else if (xg == 2) PI_UP(1, 2); else if (xg == 4) PI_UP(1, 4);
        else if (xg == 8) PI_UP(1, 8); else PI_UP(1, 16);
    } else {
        if (xg == 1) PI_UP(0, 1); else if (xg == 2) PI_UP(0, 2); else if (xg == 4) PI_UP(0, 4);
        else if (xg == 8) PI_UP(0, 8); else PI_UP(0, 16);
    }
    if (xg == 1) PI_DN(1); else if (xg == 2) PI_DN(2); else if (xg == 4) PI_DN(4);
    else if (xg == 8) PI_DN(8); else PI_DN(16);
#undef PI_UP
#undef PI_DN
    const int nq = B * (d / 4);   // four outputs per thread
    hipLaunchKernelGGL(k_union_reduce, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, s, partial, B, L.Bp,
                       d, L.G, y, count, uerr);
    return hipGetLastError();
}

hipError_t launch_bpredict(const h16* x, int B, int d, const h16* P1, const float* b1, bool relu,
                          const h16* P2, const float* b2, int r, int ffn, int hot, float thr, int32_t* idx,
                          int32_t* count, const BPredLayout& L, char* ws, char* hdr, hipStream_t s) {
    h16* h_hi = reinterpret_cast<h16*>(ws + L.h_hi);
    h16* h_lo = reinterpret_cast<h16*>(ws + L.h_lo);
    uint32_t* masks32 = reinterpret_cast<uint32_t*>(ws + L.masks32);
    float* part = reinterpret_cast<float*>(ws + L.hpart);
    uint32_t* lctr = reinterpret_cast<uint32_t*>(ws + L.lctr);
    const h16* zsrc = reinterpret_cast<const h16*>(hdr + Sync::zero);
    RingArgs ha{};
    ha.W[0] = P1;
    ha.ldw = d;
    ha.nrows = r;
    ha.X[0] = x;
    ha.ldx = d;
    ha.B = B;
    ha.K = d;
    ha.zsrc = zsrc;
    ha.part = part;
    ha.ctr = nullptr;   // pieces are added by k_bpred_hidden_finish
    RingArgs la{};
    la.W[0] = P2 + (size_t)hot * r;   // the hot prefix's rows are not read
    la.ldw = r;
    la.nrows = ffn - hot;
    la.X[0] = h_hi;
    la.X[1] = h_lo;
    la.ldx = L.ldh;
    la.B = B;
    la.K = r;
    la.zsrc = zsrc;
    la.part = part;
    la.ctr = lctr;
    const int nlctr = (ffn + kRingRows - 1) / kRingRows;
    const HiddenEpi he{b1, (int)relu, r, B, L.ldh, h_hi, h_lo};
    const int gfin = (int)(((size_t)r * B + 255) / 256);
#define PI_BH(N)                                                                                              \
    {                                                                                                         \
        const int gh = ring_grid<k_bpred_hidden<HidCfg<N>>>();                                                \
        hipLaunchKernelGGL((k_bpred_hidden<HidCfg<N>>), dim3(gh), dim3(256), 0, s, ha, he, lctr, nlctr);      \
        hipLaunchKernelGGL((k_bpred_hidden_finish<HidCfg<N>>), dim3(gfin), dim3(256), 0, s, ha, he, gh);      \
    }
    // up to 8 tokens: the hidden layer on the vector units when the group's x fits in LDS
    const int nch = d / 8;
    const int gv = (r + 3) / 4;
    const bool valu = B <= 8 && nch <= hid_valu_chunks(B <= 4 ? 4 : 8);
#define PI_BHV(TB) hipLaunchKernelGGL(k_bpred_hidden_valu<TB>, dim3(gv), dim3(256), 0, s, x, B, d, P1, he, lctr, nlctr)
#define PI_BL(N)                                                                                          \
    if (logits_tq_fits(B, r, ffn - hot)) {                                                                \
        const int nq = (B + 31) / 32, nrg = logits_tq_ranges(B);                                          \
        auto kq = r == 256 ? k_bpred_logits_tq<4> : (r == 512 ? k_bpred_logits_tq<8> : k_bpred_logits_tq<16>); \
        hipLaunchKernelGGL(kq, dim3(nq * nrg), dim3(256), 0, s, P2, ffn - hot, hot, h_hi, h_lo, L.ldh, B,  \
                           nq, nrg, b2, thr, masks32, ffn);                                                \
    } else {                                                                                              \
        hipLaunchKernelGGL((k_bpred_logits<LogCfg<N>>), dim3(ring_grid<k_bpred_logits<LogCfg<N>>>()),     \
                           dim3(256), 0, s, la, b2, thr, masks32, ffn, hot);                              \
    }
    const int xg = ring_xg(B);
    if (valu) {
        if (B <= 2) PI_BHV(2);
        else if (B <= 4) PI_BHV(4);
        else PI_BHV(8);
    }
    if (xg == 1) { if (!valu) PI_BH(1); PI_BL(1); }
    else if (xg == 2) { PI_BH(2); PI_BL(2); }
    else if (xg == 4) { PI_BH(4); PI_BL(4); }
    else if (xg == 8) { PI_BH(8); PI_BL(8); }
    else { PI_BH(16); PI_BL(16); }
#undef PI_BH
#undef PI_BHV
#undef PI_BL
    hipLaunchKernelGGL(k_bpred_compact, dim3(B), dim3(256), 0, s, masks32, ffn, hot / 32, idx, count);
    return hipGetLastError();
}

}  // namespace pi
