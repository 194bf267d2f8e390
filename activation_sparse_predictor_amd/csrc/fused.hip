// Single-token decode step, one kernel per entry point.
//
// pi_ffn_predict (B = 1):  k_predict_fused
//   workgroups [0, NA)        hidden rows, one wave per row of P1:
//                             h_k = act(P1[k].x + b1_k), published as a tagged word
//   [NA, NA + NHU)            (pi_ffn_decode_hot only) hot-prefix up rows, one
//                             wave per neuron i < n_hot: a_i, published as a tagged word
//   next NT workgroups        logits tiles of 32 neurons: collect h, stream the
//                             tile's P2 rows, z = P2 h + b2 > thr, publish the
//                             tile's 32-bit mask as a tagged word (a tile of
//                             the always-listed hot prefix exits at once)
//   the next one              gathers every mask and writes idx (ascending) and count
//   INT4 predictor            (pi_ffn_predict_q4) four logits tiles a workgroup
//                             and no gathering workgroup: each workgroup finds
//                             its place in the list by a look-back over the
//                             earlier workgroups' counts and writes its own ids;
//                             the last one writes count
//   the last T * G            (pi_ffn_decode_hot only) hot-prefix W_down: column
//                             tile x chunk of the prefix, accumulated from the
//                             prefix's a_i; the tile's last chunk adds the chunk
//                             partials in order into the FFN's extra partial slot,
//                             which the FFN kernel adds to y (its list from n_hot on)
//
// pi_ffn_sparse (B = 1):   k_sparse_fused
//   workgroups [0, NU)        up chunks, one wave per active row:
//                             a_j = act(W_up[i].x + b_up_i [, W_gate[i].x + b_gate_i]),
//                             published as a tagged word
//   workgroups [NU, NU + T*G) W_down (column tile, list chunk; chunks past
//                             ceil(count / kSChunkRows) exit at once): stage the chunk's
//                             ids, issue its row segments, collect the chunk's
//                             a_j, accumulate; the last chunk of a column tile to
//                             arrive adds the G partials in chunk order
// All up chunks precede the W_down workgroups: the up rows, which everything
// waits for, are all requested first.
//
// A tagged word is 64 bits, {epoch, 32-bit payload}, written and read with
// single-copy-atomic device-coherent accesses: a consumer polls the data
// itself, so publishing costs one store and consuming one load, with no flag
// or counter in between.  The epoch is one more than the previous launch's
// (never 0), kept in the workspace header, so a word left over from an
// earlier call never passes for a current one, also when the launches are
// replayed from a captured graph.  In predict the compaction workgroup (INT4:
// the last logits workgroup, once its look-back has resolved) stores it back:
// it runs after every other workgroup has read the epoch, because it waits for
// every tile's mask (every workgroup's count) and a tile outside the
// always-listed prefix waits for every h (when every tile lies in the prefix,
// no hidden-row workgroup is launched).  In the FFN the last chunk of each column tile stores it into that
// tile's slot, and a launch takes the oldest slot plus one: while any W_down
// workgroup of a launch is still running, its tile's slot holds the previous
// epoch.  A workgroup only waits for
// workgroups with a smaller index, which are dispatched before it, so the
// roles overlap (P1 with P2, W_up with W_down) without any risk of circular
// waiting.  Every wait is bounded: on overrun the kernel reports an error
// instead of hanging (predict: count = -1, which the FFN kernels answer with
// NaN in y; the FFN: NaN in y).
//
// Loads are issued in batches with no uniform condition around any of them:
// such a branch makes the compiler wait for every earlier load before the
// next one.  A slot past the end of its range is masked per lane, or reads a
// clamped, valid address whose value is not used; an absent bias is read
// from a zero word in the workspace.  Vector loads complete in order, so small
// loads that must be consumed early (x, ids) go out before the weight batch
// they share a counter with.
#include "common.hpp"
#include "internal.hpp"
#include "pi.h"

namespace pi {

constexpr int kWaitLimit = 1 << 16;   // polls (with a short sleep) before a wait gives up

__device__ __forceinline__ uint64_t ld_tag(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_tag(uint64_t* p, uint32_t epoch, uint32_t payload) {
    __hip_atomic_store(p, ((uint64_t)epoch << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool is_current(uint64_t v, uint32_t epoch) { return (uint32_t)(v >> 32) == epoch; }

// This launch's epoch from the stored one: plus one, skipping 0 (a zeroed
// word).  Each role requests the stored word right after the loads that gate
// its next step (never ahead of them: loads complete in order), so it adds no
// wait of its own.  It is an ordinary (cached) load: the word was last
// written by an earlier kernel, and this launch writes it only after every
// workgroup has read it.
__device__ __forceinline__ uint32_t next_epoch(uint32_t stored) {
    const uint32_t e = stored + 1u;
    return e == 0u ? 1u : e;
}

// The FFN's stored epoch: the oldest of the T per-tile slots (which differ by
// at most one launch), found across the wave with a wrap-safe minimum.  v is
// this lane's slot, slots[min(lane, T - 1)].
__device__ __forceinline__ uint32_t oldest_slot(uint32_t v) {
    const uint32_t ref = __builtin_amdgcn_readfirstlane(v);
    int dv = (int)(v - ref);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dv = min(dv, __shfl_xor(dv, off, 64));
    return ref + (uint32_t)dv;
}

// Re-read *p until it carries the epoch; false on overrun.
__device__ __forceinline__ bool poll_tag(const uint64_t* p, uint64_t& v, uint32_t epoch) {
    for (int n = 0; !is_current(v, epoch); ++n) {
        if (n == kWaitLimit) return false;
        __builtin_amdgcn_s_sleep(2);
        v = ld_tag(p);
    }
    return true;
}

// ===========================================================================
// Predict.
constexpr int kLTile = 32;    // neurons per logits tile (one 32-bit mask), 8 per wave
constexpr int kLRows = 8;     // rows per wave
constexpr int kLCols = 2;     // 64-lane chunk columns per batch: 16 P2 loads in flight per lane
static_assert(kLRows * 4 == kLTile, "4 waves per logits tile");
constexpr int kQ4Tiles = 4;   // logits tiles per workgroup of the INT4 predictor

// At the 107 VGPRs this needs, 4 workgroups fit per CU: of the 1153 of a
// 1024 x 28672 predictor, the last 129 logits tiles start as hidden rows
// retire.  Asking for 5 per CU (102 VGPRs) spills in the logits loop and
// makes the kernel half again as slow.
//
// Q4: P1 and P2 are INT4 rows (P1, P2 then point at the code bytes, two
// codes a byte, and s1, s2 at the fp16 scales of 64-weight groups); h and z
// are still accumulated in fp32.
// The hot prefix's FFN (pi_ffn_decode_hot): rows [0, n) of W_up [W_gate] and
// W_down, its activations as tagged words with their own epochs (per-tile
// slots, advanced by the FFN kernel that follows), and its chunk partials,
// which that kernel adds to y.
struct HotArgs {
    const h16* Wu;
    const float* bu;
    const h16* Wg;
    const float* bg;
    const h16* Wd;
    uint64_t* atag;
    float* partial;
    uint32_t* slots;
    int n, NHU, G, T;
};

constexpr int kHotUpMaxWG = 384;            // hot up workgroups (4 rows each, one per wave)
constexpr int kHotCols = kFusedCols;        // W_down columns per hot tile: 64 threads x 8
constexpr int kHotGroups = 4;               // row groups (waves) of a hot W_down workgroup
constexpr int kHotBatch = kHotRowsPerChunk / kHotGroups;   // rows in flight per thread
static_assert(kHotCols == 64 * 8, "one wave spans a hot tile's columns");

// Hot-prefix up rows: workgroup u takes a contiguous range of the prefix, one
// wave per neuron (the FFN kernel's up role at 256 threads).
template <int KIND>
__device__ __forceinline__ void hot_up_role(const HotArgs& H, const h16* __restrict__ x, int d, int u, float* sh,
                                            const float* __restrict__ zero) {
    constexpr bool GATED = KIND != 0;
    constexpr int UU = GATED ? 9 : 18;   // 16-byte chunks per lane per batch: a row of d <= 9216 in one
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = H.n;
    const int PU = (n + H.NHU - 1) / H.NHU;
    const int j0 = min(n, u * PU), j1 = min(n, j0 + PU);
    if (j0 >= j1) return;
    const int nch = d >> 3;
    // x to LDS by direct-to-LDS loads, 64 chunks a wave (no registers held
    // across the row batch)
    const uint32_t sxa = lds_addr(sh);
    for (int c0 = wave * 64; c0 < nch; c0 += 256) dma16(x + (size_t)min(c0 + lane, nch - 1) * 8, sxa + (uint32_t)c0 * 16u);
    wait_vm<0>();
    int i = min(j0 + wave, j1 - 1);
    const bool live = j0 + wave < j1;   // wave-uniform
    u32x4 wu[UU], wg[UU];
    auto issue = [&](int c0) {   // c0 = b0 + lane; one buffer resource per row, zeros past its end
        const uint32_t b0 = (uint32_t)(c0 - lane) * 16u;
        const auto ru = buf_rsrc(H.Wu + (size_t)i * d, (uint32_t)d * 2u);
#pragma unroll
        for (int q = 0; q < UU; ++q) wu[q] = buf_ld16_stream(ru, (uint32_t)lane * 16u, b0 + q * 1024u);
        if (GATED) {
            const auto rgp = buf_rsrc(H.Wg + (size_t)i * d, (uint32_t)d * 2u);
#pragma unroll
            for (int q = 0; q < UU; ++q) wg[q] = buf_ld16_stream(rgp, (uint32_t)lane * 16u, b0 + q * 1024u);
        }
    };
    float bu = 0.f, bgv = 0.f;
    auto issue_bias = [&]() {
        bu = *(H.bu ? H.bu + i : zero);
        if (GATED) bgv = *(H.bg ? H.bg + i : zero);
    };
    issue(lane);
    issue_bias();
    const uint32_t slot = H.slots[min(lane, H.T - 1)];
    const u32x4* sx = reinterpret_cast<const u32x4*>(sh);
    __syncthreads();
    if (!live) return;
    for (int j = j0 + wave; j < j1; j += 4) {
        if (j != j0 + wave) {
            i = j;
            issue(lane);
            issue_bias();
        }
        float au = 0.f, ag = 0.f;
        for (int c0 = lane; c0 < nch; c0 += 64 * UU) {
            if (c0 != lane) issue(c0);
#pragma unroll
            for (int q = 0; q < UU; ++q) {
                const int c = c0 + q * 64;
                if (c < nch) {
                    const u32x4 xv = sx[c];
                    au = dot8_h(wu[q], xv, au);
                    if (GATED) ag = dot8_h(wg[q], xv, ag);
                }
            }
        }
        au = group_sum<64>(au);
        if (GATED) ag = group_sum<64>(ag);
        const uint32_t epoch = next_epoch(oldest_slot(slot));
        if (lane == 0) st_tag(&H.atag[j], epoch, __float_as_uint(ffn_act<KIND>(au + bu, ag + bgv)));
    }
}

// Hot-prefix W_down: workgroup (tile, chunk) of the prefix, wave g the chunk's
// rows g, g + 4, ...; a thread holds 8 columns of 16 rows in flight, requested
// before the activations are collected.  Each wave collects its own rows'
// activations (lane q polls row q) and takes them by lane broadcast.  The
// waves are summed in LDS and the chunk partial is stored.  The FFN kernel
// that follows adds the G partials in chunk order to y and advances the
// epoch slots: a sum and an arrival count here would end this kernel with two
// more hand-offs, which cost most while the logits tiles still stream.
__device__ __forceinline__ void hot_down_role(const HotArgs& H, int d, int k, float* sh) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int rg = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int T = H.T, G = H.G, n = H.n;
    const int tile = k % T, chunk = k / T;
    const int PD = (n + G - 1) / G;
    const int j0 = min(n, chunk * PD), j1 = min(n, j0 + PD);
    const int col = tile * kHotCols + lane * 8;
    const int colc = min(col, d - 8);   // load address of a column past the end
    const int nk = (j1 - j0 - rg + kHotGroups - 1) / kHotGroups;   // this wave's rows j0 + rg + 4m
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    bool ok = true;
    uint32_t epoch = 0;
    // the slot is stable while this launch runs (the FFN kernel that follows
    // advances it), so it may be requested ahead of the rows
    const uint32_t slot = H.slots[min(lane, T - 1)];
    for (int k0 = 0; k0 == 0 || k0 < nk; k0 += kHotBatch) {
        u32x4 w[kHotBatch];
#pragma unroll
        for (int q = 0; q < kHotBatch; ++q) {
            const int r = min(j0 + rg + kHotGroups * min(k0 + q, max(nk - 1, 0)), n - 1);
            w[q] = ld16_stream(H.Wd + (size_t)r * d + colc);
        }
        if (k0 == 0) epoch = next_epoch(oldest_slot(slot));
        const int q = lane & (kHotBatch - 1);
        const int jr = min(j0 + rg + kHotGroups * (k0 + q), n - 1);
        uint64_t v = ld_tag(&H.atag[jr]);
        float a = 0.f;
        if (lane < kHotBatch && k0 + q < nk) {
            ok = poll_tag(&H.atag[jr], v, epoch) && ok;
            a = __uint_as_float((uint32_t)v);
        }
#pragma unroll
        for (int m = 0; m < kHotBatch; ++m)
            if (k0 + m < nk) axpy8(acc, __shfl(a, m, 64), w[m]);
    }
    ok = __syncthreads_and(ok);
    float* s_red = sh;   // kHotGroups x kHotCols fp32
    *reinterpret_cast<f32x4*>(&s_red[rg * kHotCols + lane * 8]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(&s_red[rg * kHotCols + lane * 8 + 4]) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kHotCols / 256; ++e) {
        const int c = tid + 256 * e, gc = tile * kHotCols + c;
        if (gc < d) {
            float v = 0.f;
#pragma unroll
            for (int g = 0; g < kHotGroups; ++g) v += s_red[g * kHotCols + c];
            st_coherent(&H.partial[(size_t)chunk * d + gc], ok ? v : __builtin_nanf(""));
        }
    }
}

// The ordered list, written by the logits workgroups themselves with a
// single-pass prefix sum over their counts (decoupled look-back: Merrill and
// Garland, "Single-pass Parallel Prefix Scan with Decoupled Look-back", 2016).
// Workgroup w owns tiles [w TPW, w TPW + TPW).  It publishes in desc[w] first
// its own count (AGG), then the count of every neuron up to its last tile
// (INC, the flag bit set).  It sums its predecessors' descriptors back to the
// nearest INC, 256 of them per round (one a thread), and writes its neurons'
// ids at their positions.  The last workgroup writes the count and stores the
// epoch: an INC stands for every workgroup before it, so by then every one
// that reads the epoch has read it.  Workgroups below w0 hold only tiles of
// the always-listed prefix: their counts are known (32 a tile), they publish
// nothing and read no epoch.  ERR marks a wait that ran out, here or before;
// it passes down the chain and makes the count -1.  The INT4 predictor uses
// it: its workgroups (four tiles each) are all resident at once.  With one
// tile a workgroup (the fp16 predictor, more workgroups than slots) the
// look-back waits held slots that later tiles needed and made the step
// slower, so that predictor keeps its gathering workgroup.
constexpr uint32_t kDescInc = 1u << 31, kDescErr = 1u << 30, kDescVal = kDescErr - 1u;
// Descriptors sit 128 bytes apart: with every workgroup polling its
// predecessors', eight to a cache line made the step 0.7 us slower.
constexpr int kDescStride = 16;
static_assert(kQ4Tiles == 4 && kDescStride * 8 == 128, "fused_pred_layout sizes the descriptors so");

template <int TPW>
__device__ __forceinline__ void list_prefix_tiles(int w, int NT, int NW, int32_t* __restrict__ idx,
                                                  int32_t* __restrict__ count, uint32_t* __restrict__ epoch_word) {
    const int j0 = w * TPW * kLTile, j1 = min(w * TPW + TPW, NT) * kLTile;
    for (int j = j0 + (int)threadIdx.x; j < j1; j += 256) idx[j] = j;
    if (w == NW - 1 && threadIdx.x == 0) {
        count[0] = j1;
        st_flag(epoch_word, next_epoch(*epoch_word));
    }
}

// s_mask: the TPW tile masks (LDS, written before a barrier); ok: this
// workgroup's own waits held (block-uniform); s_red: 8 words of LDS.
template <int TPW>
__device__ __forceinline__ void list_tiles(int w, int w0, int NW, const uint32_t* s_mask, bool ok, uint32_t epoch,
                                           uint64_t* __restrict__ desc, int32_t* __restrict__ idx,
                                           int32_t* __restrict__ count, uint32_t* __restrict__ epoch_word,
                                           uint32_t* s_red, int ffn) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    uint32_t agg = 0;
#pragma unroll
    for (int q = 0; q < TPW; ++q) agg += (uint32_t)__popc(s_mask[q]);
    uint32_t flags = ok ? 0u : kDescErr;
    uint32_t excl = (uint32_t)(w0 * TPW * kLTile);
    if (w > w0) {
        if (tid == 0) st_tag(&desc[(size_t)w * kDescStride], epoch, flags | agg);
        uint32_t sum = 0;
        for (int base = w;; base -= 256) {
            const int j = base - 1 - tid;   // thread 0: the nearest predecessor
            const bool in = j >= w0;
            uint64_t v = ld_tag(&desc[(size_t)max(j, w0) * kDescStride]);
            bool good = true;
            if (in) good = poll_tag(&desc[(size_t)j * kDescStride], v, epoch);
            const uint32_t lo = (uint32_t)v;
            const uint64_t inc = __ballot(in && good && (lo & kDescInc));
            if (lane == 0) s_red[wave] = inc ? (uint32_t)(wave * 64 + __builtin_ctzll(inc)) : 256u;
            __syncthreads();
            const uint32_t first = min(min(s_red[0], s_red[1]), min(s_red[2], s_red[3]));
            // the descriptors nearer than the nearest INC, and that INC
            const bool take = in && (uint32_t)tid <= first;
            uint32_t val = take ? (lo & kDescVal) : 0u;
            uint32_t bad = take && (!good || (lo & kDescErr)) ? 1u : 0u;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                val += __shfl_xor(val, off, 64);
                bad |= __shfl_xor(bad, off, 64);
            }
            __syncthreads();
            if (lane == 0) {
                s_red[wave] = val;
                s_red[4 + wave] = bad;
            }
            __syncthreads();
            sum += s_red[0] + s_red[1] + s_red[2] + s_red[3];
            if (s_red[4] | s_red[5] | s_red[6] | s_red[7]) flags = kDescErr;
            __syncthreads();   // s_red is the next round's
            if (first < 256u) {   // an INC counts every neuron before it
                excl = sum;
                break;
            }
            if (base - 256 <= w0) {   // back to the prefix workgroups
                excl += sum;
                break;
            }
        }
    }
    if (tid == 0) st_tag(&desc[(size_t)w * kDescStride], epoch, flags | kDescInc | min(excl + agg, kDescVal));
    if (!flags && tid < TPW * kLTile) {
        const int q = tid >> 5, bit = tid & 31;
        const uint32_t m = s_mask[q];
        if ((m >> bit) & 1u) {
            uint32_t pos = excl + (uint32_t)__popc(m & ((1u << bit) - 1u));
#pragma unroll
            for (int q2 = 0; q2 < TPW - 1; ++q2)
                if (q2 < q) pos += (uint32_t)__popc(s_mask[q2]);
            if (pos < (uint32_t)ffn) idx[pos] = (w * TPW + q) * kLTile + bit;
        }
    }
    if (w == NW - 1 && tid == 0) {
        count[0] = flags ? -1 : (int32_t)(excl + agg);
        st_flag(epoch_word, epoch);
    }
}

// Logits tiles of the INT4 predictor, kQ4Tiles per workgroup.  INT4 rows
// of r / 32 chunks (16 bytes, 32 codes); half-wave hf of wave w takes rows
// 32 t + 8 w + hf + 2m (m < 4) of each of its tiles t, lane chunk
// c = (lane & 31) + 32n.  The first column batch of every tile is requested
// at once, then h is read (after the rows, so it is fresh), then each h chunk
// and its sum serve the four rows of every tile.  One h collection per four
// tiles (a quarter of the workgroups polling h, and four tiles' rows in
// flight during the wait).
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Bytes 2 UP and 2 UP + 1 of v, each below 16, as floats u * byte.  The fp8
// (e4m3) conversion reads such a byte as a multiple of the format's smallest
// step u (a power of two: subnormals, then the first binade, same spacing), so
// no value is rounded; one instruction converts two codes.
template <bool UP>
__device__ __forceinline__ f32x2 code_pair(uint32_t v) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)v, UP);
}
__device__ __forceinline__ void q4_logits_tiles(int tw, const uint8_t* __restrict__ q2, const h16* __restrict__ s2,
                                                const float* __restrict__ b2, int ffn, int r, float thr, int hot,
                                                const uint64_t* __restrict__ htag, uint64_t* __restrict__ desc,
                                                uint32_t* __restrict__ epoch_word, int32_t* __restrict__ idx,
                                                int32_t* __restrict__ count, const float* __restrict__ zero, float* sh,
                                                uint32_t* s_act, uint32_t* s_mask, uint32_t* s_red) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5;
    const int NT = (ffn + kLTile - 1) / kLTile;
    const int NW = (NT + kQ4Tiles - 1) / kQ4Tiles;
    const int w0 = min(hot / kLTile, NT) / kQ4Tiles;   // workgroups holding only prefix tiles
    const int t0 = tw * kQ4Tiles;
    // every tile of this workgroup in the always-listed prefix: no P2 row and
    // no wait for h
    if (min(t0 + kQ4Tiles, NT) * kLTile <= hot) {
        list_prefix_tiles<kQ4Tiles>(tw, NT, NW, idx, count, epoch_word);
        return;
    }
    const int ncw = r >> 5, ng = r >> 6;
    const int NB = (ncw + 31) >> 5;   // column batches (1 for r <= 1024)
    auto rowof = [&](int qt, int m) { return min((t0 + qt) * kLTile + wave * kLRows + hf + 2 * m, ffn - 1); };
    const int c0 = lane & 31;
    const float inv_u = 8.f / code_pair<false>(8u).x;   // 1 / u
    // first batch of every tile (a lane past the row end reads its last chunk:
    // valid, unused), and lane k < 8's bias of row 8w + k of every tile
    u32x4 w[kQ4Tiles][4];
    h16 sc[kQ4Tiles][4];
    float bias[kQ4Tiles];
    {
        const int cl = min(c0, ncw - 1);
#pragma unroll
        for (int qt = 0; qt < kQ4Tiles; ++qt) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int rr = rowof(qt, m);
                w[qt][m] = ld16_stream(q2 + (size_t)rr * (r / 2) + (size_t)cl * 16);
                sc[qt][m] = s2[(size_t)rr * ng + (cl >> 1)];
            }
            bias[qt] = *(b2 ? b2 + min((t0 + qt) * kLTile + wave * kLRows + (lane & (kLRows - 1)), ffn - 1) : zero);
        }
    }
    // h, once the rows are in (a poll issued behind them would come back with
    // them, holding h as it was when the poll was served)
    wait_own_memory();
    const uint32_t epoch = next_epoch(*epoch_word);
    bool ok = true;
    for (int i0 = tid; i0 < r; i0 += 1024) {
        uint64_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = ld_tag(&htag[i0 + q * 256]);   // padded to 1024 words
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = i0 + q * 256;
            if (i < r) {
                ok = poll_tag(&htag[i], v[q], epoch) && ok;
                sh[i] = __uint_as_float((uint32_t)v[q]);
            }
        }
    }
    ok = __syncthreads_and(ok);
    float a4[kQ4Tiles][4];
#pragma unroll
    for (int qt = 0; qt < kQ4Tiles; ++qt)
#pragma unroll
        for (int m = 0; m < 4; ++m) a4[qt][m] = 0.f;
    for (int n = 0; n < NB; ++n) {
        const int c = c0 + 32 * n;
        if (n > 0) {   // r > 1024: the later batches, one at a time
            const int cl = min(c, ncw - 1);
#pragma unroll
            for (int qt = 0; qt < kQ4Tiles; ++qt)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int rr = rowof(qt, m);
                    w[qt][m] = ld16_stream(q2 + (size_t)rr * (r / 2) + (size_t)cl * 16);
                    sc[qt][m] = s2[(size_t)rr * ng + (cl >> 1)];
                }
        }
        if (c < ncw) {
            const f32x4* hp = reinterpret_cast<const f32x4*>(sh + c * 32);
            float hv[32];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const f32x4 v = hp[q];
                hv[4 * q] = v.x;
                hv[4 * q + 1] = v.y;
                hv[4 * q + 2] = v.z;
                hv[4 * q + 3] = v.w;
            }
            // sum_k (code_k - 8) h_k = sum_k code_k h_k - 8 sum_k h_k: the
            // chunk's sum of h is taken once for all its rows
            float hs = 0.f;
#pragma unroll
            for (int k = 0; k < 32; ++k) hs += hv[k];
            const float nhs8 = -8.f * hs;
            float p[kQ4Tiles][4];
#pragma unroll
            for (int qt = 0; qt < kQ4Tiles; ++qt)
#pragma unroll
                for (int m = 0; m < 4; ++m) p[qt][m] = 0.f;
            // word e of every row in turn (sixteen independent sums); each
            // nibble field becomes a byte (lo: weights 8e + 2j, hi: 8e + 2j + 1)
            // and each byte pair converts in one instruction to u * code
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int qt = 0; qt < kQ4Tiles; ++qt)
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const uint32_t cw = e == 0 ? w[qt][m].x : e == 1 ? w[qt][m].y : e == 2 ? w[qt][m].z : w[qt][m].w;
                        const uint32_t lo = cw & 0x0F0F0F0Fu;
                        const uint32_t hi = (cw >> 4) & 0x0F0F0F0Fu;
                        const f32x2 l01 = code_pair<false>(lo), l23 = code_pair<true>(lo);
                        const f32x2 h01 = code_pair<false>(hi), h23 = code_pair<true>(hi);
                        float s = p[qt][m];
                        s = fmaf(l01.x, hv[8 * e + 0], s);
                        s = fmaf(h01.x, hv[8 * e + 1], s);
                        s = fmaf(l01.y, hv[8 * e + 2], s);
                        s = fmaf(h01.y, hv[8 * e + 3], s);
                        s = fmaf(l23.x, hv[8 * e + 4], s);
                        s = fmaf(h23.x, hv[8 * e + 5], s);
                        s = fmaf(l23.y, hv[8 * e + 6], s);
                        s = fmaf(h23.y, hv[8 * e + 7], s);
                        p[qt][m] = s;
                    }
            // p = u * sum_k code_k h_k exactly (u a power of two)
#pragma unroll
            for (int qt = 0; qt < kQ4Tiles; ++qt)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    a4[qt][m] = fmaf((float)sc[qt][m], fmaf(p[qt][m], inv_u, nhs8), a4[qt][m]);
        }
    }
#pragma unroll
    for (int qt = 0; qt < kQ4Tiles; ++qt) {
        const int tile = t0 + qt;
        if (tile >= NT) {   // past the last tile
            if (tid == 0) s_mask[qt] = 0u;
            continue;
        }
        float zk = 0.f;   // lane k < 8: row k is half k & 1's row 2m + (k & 1), m = k / 2
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float z = __shfl(group_sum<32>(a4[qt][m]), (lane & 1) << 5, 64);
            if (((lane & (kLRows - 1)) >> 1) == m) zk = z;
        }
        if ((tile + 1) * kLTile <= hot) {   // a prefix tile: every neuron listed
            if (tid == 0) s_mask[qt] = ~0u;
            continue;
        }
        const int row0 = tile * kLTile + wave * kLRows;
        if (lane < kLRows) s_act[wave * kLRows + lane] = (row0 + lane < ffn) && (zk + bias[qt] > thr);
        __syncthreads();
        if (wave == 0) {
            const uint64_t mk = __ballot(lane < kLTile && s_act[lane & (kLTile - 1)] != 0u);
            if (lane == 0) s_mask[qt] = (uint32_t)mk;
        }
        __syncthreads();   // s_act is the next tile's
    }
    __syncthreads();
    list_tiles<kQ4Tiles>(tw, w0, NW, s_mask, ok, epoch, desc, idx, count, epoch_word, s_red, ffn);
}

template <bool Q4, int HK>
__global__ __launch_bounds__(256) void k_predict_fused(const h16* __restrict__ x, int d,
                                                       const h16* __restrict__ P1,
                                                       const float* __restrict__ b1, int relu, int r,
                                                       const h16* __restrict__ P2,
                                                       const float* __restrict__ b2, int ffn, float thr,
                                                       uint64_t* __restrict__ htag, uint64_t* __restrict__ desc,
                                                       uint32_t* __restrict__ epoch_word, int32_t* __restrict__ idx,
                                                       int32_t* __restrict__ count, const float* __restrict__ zero,
                                                       int hot, int NA, const h16* __restrict__ s1,
                                                       const h16* __restrict__ s2, HotArgs H) {
    extern __shared__ float sh[];  // hidden role: x (d fp16); logits role: h (r fp32)
    __shared__ uint32_t s_act[kLTile];
    __shared__ uint32_t s_mask[kQ4Tiles];
    __shared__ uint32_t s_red[8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int NT = (ffn + kLTile - 1) / kLTile;
    const int NHU = HK >= 0 ? H.NHU : 0;
    const int b = blockIdx.x;
    const int lg0 = NA + NHU;   // first logits tile
    // The hot W_down workgroups come last: placed among the logits tiles (from
    // any position) they held slots the tiles needed and made the step slower.
    if constexpr (HK >= 0) {
        if (b >= NA && b < lg0) {
            hot_up_role<HK>(H, x, d, b - NA, sh, zero);
            return;
        }
        if (b > lg0 + NT) {
            hot_down_role(H, d, b - (lg0 + NT + 1), sh);
            return;
        }
    }
    const int tile = b - lg0;

    if (b < NA) {
        // ---------------- hidden rows
        const int row = blockIdx.x * 4 + wave;
        const bool valid = row < r;
        const h16* prow = P1 + (size_t)min(row, r - 1) * d;
        const int nch = d >> 3;
        u32x4 xs[4];   // x chunks tid + 256 q, requested ahead of the P1 rows
#pragma unroll
        for (int q = 0; q < 4; ++q) xs[q] = ld16(x + (size_t)min(tid + q * 256, nch - 1) * 8);
        if constexpr (Q4) {
            // INT4 row: d / 32 chunks of 16 bytes (32 codes, half a scale group)
            constexpr int UH = 4;   // chunks per lane per batch
            const uint8_t* qrow = reinterpret_cast<const uint8_t*>(P1) + (size_t)min(row, r - 1) * (d / 2);
            const h16* srow = s1 + (size_t)min(row, r - 1) * (d >> 6);
            const int ncw = d >> 5;
            // Slots past the row end read its last chunk (valid, unused): no
            // branch around a load, and each scale stays fp16 until its use, so
            // no load waits for another.
            u32x4 w[UH];
            h16 sc[UH];
            auto issue = [&](int c0) {
#pragma unroll
                for (int u = 0; u < UH; ++u) {
                    const int c = min(c0 + u * 64, ncw - 1);
                    w[u] = ld16_stream(qrow + (size_t)c * 16);
                    sc[u] = srow[c >> 1];
                }
            };
            issue(lane);
            const uint32_t stored = *epoch_word;
            const float bias = *(b1 ? b1 + min(row, r - 1) : zero);
            u32x4* sx = reinterpret_cast<u32x4*>(sh);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (tid + q * 256 < nch) sx[tid + q * 256] = xs[q];
            for (int i = tid + 1024; i < nch; i += 256) sx[i] = ld16(x + (size_t)i * 8);   // d > 8192
            __syncthreads();
            float acc = 0.f;
            for (int c0 = lane; c0 < ncw; c0 += 64 * UH) {
                if (c0 != lane) issue(c0);
#pragma unroll
                for (int u = 0; u < UH; ++u) {
                    const int c = c0 + u * 64;
                    if (c < ncw) {
                        const uint32_t cw[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
                        float p = 0.f;
#pragma unroll
                        for (int e = 0; e < 4; ++e) p = dot8_q4(cw[e], sx[c * 4 + e], p);
                        acc = fmaf((float)sc[u], p, acc);
                    }
                }
            }
            const float sum = group_sum<64>(acc) + bias;
            const uint32_t epoch = next_epoch(stored);
            if (valid && lane == 0) st_tag(&htag[row], epoch, __float_as_uint(relu ? fmaxf(sum, 0.f) : sum));
            return;
        }
        // 18 chunks per lane: a row of d <= 9216 is requested in one round; one
        // buffer resource per row, chunks past its end load zeros
        constexpr int HU = 18;
        const auto rp = buf_rsrc(prow, (uint32_t)d * 2u);
        u32x4 w[HU];
#pragma unroll
        for (int u = 0; u < HU; ++u) w[u] = buf_ld16_stream(rp, (uint32_t)lane * 16u, u * 1024u);
        const uint32_t stored = *epoch_word;
        const float bias = *(b1 ? b1 + min(row, r - 1) : zero);
        u32x4* sx = reinterpret_cast<u32x4*>(sh);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (tid + q * 256 < nch) sx[tid + q * 256] = xs[q];
        for (int i = tid + 1024; i < nch; i += 256) sx[i] = ld16(x + (size_t)i * 8);   // d > 8192
        __syncthreads();
        float acc = 0.f;
        for (int c0 = lane; c0 < nch; c0 += 64 * HU) {
            if (c0 != lane) {
#pragma unroll
                for (int u = 0; u < HU; ++u) w[u] = buf_ld16_stream(rp, (uint32_t)lane * 16u, (uint32_t)(c0 - lane + u * 64) * 16u);
            }
#pragma unroll
            for (int u = 0; u < HU; ++u) {
                const int c = c0 + u * 64;
                if (c < nch) acc = dot8_h(w[u], sx[c], acc);
            }
        }
        const float s = group_sum<64>(acc) + bias;
        const uint32_t epoch = next_epoch(stored);
        if (valid && lane == 0) st_tag(&htag[row], epoch, __float_as_uint(relu ? fmaxf(s, 0.f) : s));
        return;
    }

    if (!Q4 && b == lg0 + NT) {
        // ---------------- ordered compaction.  The always-listed prefix [0, hot)
        // is written first, by every thread in turn (coalesced, no mask read).
        // The other tiles go 256 per round, in tile order, thread k taking tile
        // k: one block-wide scan and one tile's ids per thread per round.  The
        // tiles publish roughly in order, so the rounds keep pace with them and
        // only the last round's scan and writes follow the last mask (the dense
        // tiles right after a hot-first prefix are long written by then).  The
        // next round's mask is requested before this round's ids go out.
        const uint32_t epoch = next_epoch(*epoch_word);
        for (int j = tid; j < hot; j += 256) idx[j] = j;
        uint32_t base = (uint32_t)hot;
        bool good = true;
        const int tb = hot / kLTile;
        uint64_t mnext = ld_tag(&desc[min(tb + tid, NT - 1)]);
        for (int t0 = tb, k = 0; t0 < NT; t0 += 256, ++k) {
            const int t = t0 + tid;
            uint64_t m = mnext;
            mnext = ld_tag(&desc[min(t + 256, NT - 1)]);
            uint32_t bits = 0u;
            if (t < NT) {
                if (poll_tag(&desc[t], m, epoch)) bits = (uint32_t)m;
                else good = false;
            }
            const uint32_t c = (uint32_t)__popc(bits);
            uint32_t incl = c;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t v = __shfl_up(incl, off, 64);
                if (lane >= off) incl += v;
            }
            uint32_t* sw = s_red + (k & 1) * 4;   // alternate halves: one barrier a round
            if (lane == 63) sw[wave] = incl;
            __syncthreads();
            uint32_t pos = base + incl - c;
            for (int w2 = 0; w2 < wave; ++w2) pos += sw[w2];
            base += sw[0] + sw[1] + sw[2] + sw[3];
            while (bits) {
                idx[pos++] = t * kLTile + __builtin_ctz(bits);
                bits &= bits - 1u;
            }
        }
        good = __syncthreads_and(good);
        if (tid == 0) {
            count[0] = good ? (int32_t)base : -1;
            // every other workgroup that reads the epoch has read it: each
            // logits tile outside the prefix has published its mask, after
            // every hidden row its h (without such a tile no hidden row runs;
            // the prefix's tiles read nothing)
            st_flag(epoch_word, epoch);
        }
        return;
    }

    if constexpr (Q4) {
        q4_logits_tiles(tile, reinterpret_cast<const uint8_t*>(P2), s2, b2, ffn, r, thr, hot, htag, desc, epoch_word,
                        idx, count, zero, sh, s_act, s_mask, s_red);
        return;
    }
    // ---------------- logits tile: wave w owns neurons tile*32 + 8w + k (k < 8); lane l
    // takes chunks l + 64m of all eight rows, so an h chunk read from LDS serves
    // eight rows
    if ((tile + 1) * kLTile <= hot) {
        // a tile of the always-listed hot prefix (hot is a multiple of 32):
        // every neuron on, which the compaction writes without a mask; no P2
        // row read, no wait for h
        return;
    }
    const int row0 = tile * kLTile + wave * kLRows;   // wave-uniform
    const int nch = r >> 3;
    const int M = (nch + 63) / 64;                     // chunk columns per lane
    const h16* prow[kLRows];
#pragma unroll
    for (int k = 0; k < kLRows; ++k) prow[k] = P2 + (size_t)min(row0 + k, ffn - 1) * r;
    float bias = 0.f;   // lane k < 8: b2 of row row0 + k
    uint32_t epoch = 0;
    float acc[kLRows];
#pragma unroll
    for (int k = 0; k < kLRows; ++k) acc[k] = 0.f;
    bool ok = true;
    // h (and b2) are read once the tile's first batch of P2 rows has arrived.
    // Loads return in order, so a poll issued behind the batch would come back
    // with it, holding what h was when the poll was served, long before; read
    // after the batch it is fresh, and the hidden rows (which compete with P2
    // for bandwidth from the start) are long done by then.
    bool have_h = false;
    auto check_round = [&](int i0, uint64_t (&v)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = i0 + q * 256;
            if (i < r) {
                ok = poll_tag(&htag[i], v[q], epoch) && ok;
                sh[i] = __uint_as_float((uint32_t)v[q]);
            }
        }
    };
    auto collect_h = [&]() {
        uint64_t v[4];
        epoch = next_epoch(*epoch_word);
        bias = *(b2 ? b2 + min(row0 + (lane & (kLRows - 1)), ffn - 1) : zero);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = ld_tag(&htag[tid + q * 256]);   // padded to 1024 words
        check_round(tid, v);   // outside any loop: a loop header would wait for the P2 batch first
        for (int i0 = tid + 1024; i0 < r; i0 += 1024) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = ld_tag(&htag[i0 + q * 256]);
            check_round(i0, v);
        }
        ok = __syncthreads_and(ok);
        have_h = true;
    };
    // z of row row0 + k in lane k < 8 (with the bias): the tile's 32-bit mask
    auto publish = [&](float zk) {
        if (lane < kLRows) s_act[wave * kLRows + lane] = (row0 + lane < ffn) && (zk + bias > thr);
        __syncthreads();
        if (wave == 0) {
            const uint64_t m = __ballot(lane < kLTile && s_act[lane & (kLTile - 1)] != 0u);
            if (lane == 0 && ok) st_tag(&desc[tile], epoch, (uint32_t)m);
        }
    };
    auto accumulate = [&](const u32x4 (&w)[kLRows][kLCols], int m0) {
#pragma unroll
        for (int m = 0; m < kLCols; ++m) {
            const int c = lane + (m0 + m) * 64;
            if (c < nch) {
                const f32x4* hp = reinterpret_cast<const f32x4*>(sh + c * 8);
                const f32x4 h0 = hp[0], h1 = hp[1];
                const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
                for (int k = 0; k < kLRows; ++k) acc[k] = dot8_hf(w[k][m], hv, acc[k]);
            }
        }
    };
    int m0 = 0;
    for (; (m0 + kLCols) * 64 <= nch; m0 += kLCols) {   // full batches: every lane in range
        u32x4 w[kLRows][kLCols];
#pragma unroll
        for (int k = 0; k < kLRows; ++k)
#pragma unroll
            for (int m = 0; m < kLCols; ++m) w[k][m] = ld16_stream(prow[k] + (size_t)(lane + (m0 + m) * 64) * 8);
        if (!have_h) {
            wait_own_memory();
            collect_h();
        }
        accumulate(w, m0);
    }
    if (m0 < M) {   // the last, partial batch: lanes past the row end are masked
        u32x4 w[kLRows][kLCols];
#pragma unroll
        for (int k = 0; k < kLRows; ++k)
#pragma unroll
            for (int m = 0; m < kLCols; ++m) {
                const int c = lane + (m0 + m) * 64;
                if (c < nch) w[k][m] = ld16_stream(prow[k] + (size_t)c * 8);
            }
        if (!have_h) {
            wait_own_memory();
            collect_h();
        }
        accumulate(w, m0);
    }
    float zk = 0.f;   // lane k < 8: z of row row0 + k
#pragma unroll
    for (int k = 0; k < kLRows; ++k) {
        const float z = group_sum<64>(acc[k]);
        if ((lane & (kLRows - 1)) == k) zk = z;
    }
    publish(zk);
}

// ===========================================================================
// Sparse FFN.
constexpr int kSThreads = 512;                       // 8 waves
constexpr int kSColThreads = kFusedCols / 8;         // column threads of a W_down tile (8 fp16 each)
constexpr int kSGroups = kSThreads / kSColThreads;   // row groups per W_down workgroup
constexpr int kSBatch = 16;                          // W_down rows in flight per thread
constexpr int kSChunkRows = kSGroups * kSBatch;      // list entries of a chunk that fill one batch per group
constexpr int kSWindow = 2048;                       // list entries staged in LDS at a time
static_assert(kSColThreads * kSGroups == kSThreads, "tile shape");
static_assert(kFusedCols <= kSThreads, "one reduction column per thread");

// Q4: the rows are INT4 (pi_quantize_rows: 4-bit codes, d / 2 bytes a row, and
// one fp16 scale per 64 weights in su / sg / sd); the weight pointers then
// point at the codes.  The up role takes 16-byte code chunks (32 weights)
// with their scale, the W_down role one 32-bit code word (8 columns) and one
// scale per row.
template <int KIND, bool Q4 = false>
__global__ __launch_bounds__(kSThreads) void k_sparse_fused(const h16* __restrict__ x, int d, int ffn,
                                                            const h16* __restrict__ Wup,
                                                            const float* __restrict__ bup,
                                                            const h16* __restrict__ Wg,
                                                            const float* __restrict__ bg,
                                                            const h16* __restrict__ Wd,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ count, int skip, int NU,
                                                            int T, int G, uint64_t* __restrict__ atag,
                                                            float* __restrict__ partial,
                                                            uint32_t* __restrict__ ctr, uint32_t* __restrict__ slots,
                                                            float* __restrict__ y,
                                                            const float* __restrict__ zero,
                                                            const h16* __restrict__ su = nullptr,
                                                            const h16* __restrict__ sg = nullptr,
                                                            const h16* __restrict__ sd = nullptr,
                                                            const float* __restrict__ hpart = nullptr, int hG = 0,
                                                            uint32_t* __restrict__ hslots = nullptr, int hT = 0) {
    // up role: x (d fp16); W_down role: row-group partials, window ids and activations
    __shared__ __align__(16) char s_mem[kSGroups * kFusedCols * 4 + kSWindow * 8];
    static_assert(sizeof(s_mem) >= PI_MAX_D * 2, "x does not fit the up role's LDS");
    u32x4* s_x = reinterpret_cast<u32x4*>(s_mem);
    float(*s_red)[kFusedCols] = reinterpret_cast<float(*)[kFusedCols]>(s_mem);
    int32_t* s_row = reinterpret_cast<int32_t*>(s_mem + kSGroups * kFusedCols * 4);
    float* s_a = reinterpret_cast<float*>(s_mem + kSGroups * kFusedCols * 4 + kSWindow * 4);
    __shared__ int s_flag;
    constexpr bool REGLU = KIND != 0;   // gated: a W_gate row per neuron (ReGLU, SwiGLU)
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int craw = count[0];   // negative: the predictor's overrun report, answered with NaN in y
    const int cnt = min(max(craw, 0), ffn);
    // list positions [0, sk) are the hot prefix, computed by the predictor's kernel
    // (skip > 0); this launch takes [sk, cnt) and adds the prefix's sum to y
    const int sk = min(max(skip, 0), cnt);
    const int nl = cnt - sk;
    const int PU = (nl + NU - 1) / NU;   // list positions per up chunk

    if ((int)blockIdx.x < NU) {
        // ---------------- up chunk: one wave per active row
        const int u = blockIdx.x;
        const int j0 = sk + min(nl, u * PU), j1 = min(cnt, j0 + PU);
        if (j0 >= j1) return;
        // 16-byte chunks per lane per batch: an fp16 row of d <= 9216 goes out in one round
        constexpr int UU = Q4 ? (REGLU ? 2 : 4) : (REGLU ? 9 : 18);
        const int nch = d >> 3;                     // 8-weight x chunks
        const int ncw = Q4 ? d >> 5 : nch;          // 16-byte weight chunks of a row
        const int ng = d >> 6;                      // INT4 scale groups of a row
        int j = j0 + wave;
        int i = 0;
        u32x4 wu[UU], wg[UU];
        h16 cu[UU], cg[UU];   // INT4: the chunks' scales, converted at use
        auto issue = [&](int c0) {   // c0 = b0 + lane, b0 the batch's first chunk (uniform)
            if constexpr (Q4) {
                // slots past the row end read its last chunk (valid, unused):
                // no branch around a load, so no load waits for another
                const uint8_t* ru = reinterpret_cast<const uint8_t*>(Wup) + (size_t)i * (d / 2);
                const uint8_t* rg = REGLU ? reinterpret_cast<const uint8_t*>(Wg) + (size_t)i * (d / 2) : nullptr;
#pragma unroll
                for (int q = 0; q < UU; ++q) {
                    const int c = min(c0 + q * 64, ncw - 1);
                    wu[q] = ld16_stream(ru + (size_t)c * 16);
                    cu[q] = su[(size_t)i * ng + (c >> 1)];
                    if (REGLU) {
                        wg[q] = ld16_stream(rg + (size_t)c * 16);
                        cg[q] = sg[(size_t)i * ng + (c >> 1)];
                    }
                }
            } else {
                // one buffer resource per row: chunks past the row end load zeros
                const auto ru = buf_rsrc(Wup + (size_t)i * d, (uint32_t)d * 2u);
                const uint32_t b0 = (uint32_t)(c0 - lane) * 16u;
#pragma unroll
                for (int q = 0; q < UU; ++q) wu[q] = buf_ld16_stream(ru, (uint32_t)lane * 16u, b0 + q * 1024u);
                if (REGLU) {
                    const auto rg = buf_rsrc(Wg + (size_t)i * d, (uint32_t)d * 2u);
#pragma unroll
                    for (int q = 0; q < UU; ++q) wg[q] = buf_ld16_stream(rg, (uint32_t)lane * 16u, b0 + q * 1024u);
                }
            }
        };
        float bu = 0.f, bgv = 0.f;   // the row's biases, requested with its weights
        auto issue_bias = [&]() {
            bu = *(bup ? bup + i : zero);
            if (REGLU) bgv = *(bg ? bg + i : zero);
        };
        // x goes to LDS by direct-to-LDS loads (no registers held across the
        // row batch: a d = 9216 row then fits one batch of 18 chunks per
        // lane).  The row ids are needed before the rows can go out, so
        // waiting for both costs nothing the rows did not wait for anyway.
        const uint32_t sxa = lds_addr(s_x);
        for (int c0 = wave * 64; c0 < nch; c0 += kSThreads)   // 64 chunks a wave, lane l chunk c0 + l
            dma16(x + (size_t)min(c0 + lane, nch - 1) * 8, sxa + (uint32_t)c0 * 16u);
        const bool live = j < j1;   // wave-uniform
        // the row id is wave-uniform: kept in a scalar register, the row's loads
        // take one base and per-lane offsets
        i = __builtin_amdgcn_readfirstlane(min(max(idx[min(j, j1 - 1)], 0), ffn - 1));
        issue_bias();
        wait_vm<0>();
        issue(lane);
        const uint32_t slot = slots[min(lane, T - 1)];
        __syncthreads();
        if (!live) return;
        bool first = true;
        for (; j < j1; j += kSThreads / 64) {
            if (!first) {
                i = __builtin_amdgcn_readfirstlane(min(max(idx[j], 0), ffn - 1));
                issue(lane);
                issue_bias();
            }
            first = false;
            float au = 0.f, ag = 0.f;
            for (int c0 = lane; c0 < ncw; c0 += 64 * UU) {
                if (c0 != lane) issue(c0);
#pragma unroll
                for (int q = 0; q < UU; ++q) {
                    const int c = c0 + q * 64;
                    if (c < ncw) {
                        if constexpr (Q4) {
                            const uint32_t cw[4] = {wu[q].x, wu[q].y, wu[q].z, wu[q].w};
                            const uint32_t gw[4] = {wg[q].x, wg[q].y, wg[q].z, wg[q].w};
                            float pu = 0.f, pg = 0.f;
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const u32x4 xv = s_x[c * 4 + e];
                                pu = dot8_q4(cw[e], xv, pu);
                                if (REGLU) pg = dot8_q4(gw[e], xv, pg);
                            }
                            au = fmaf((float)cu[q], pu, au);
                            if (REGLU) ag = fmaf((float)cg[q], pg, ag);
                        } else {
                            const u32x4 xv = s_x[c];
                            au = dot8_h(wu[q], xv, au);
                            if (REGLU) ag = dot8_h(wg[q], xv, ag);
                        }
                    }
                }
            }
            au = group_sum<64>(au);
            if (REGLU) ag = group_sum<64>(ag);
            const uint32_t epoch = next_epoch(oldest_slot(slot));
            if (lane == 0) {
                st_tag(&atag[j], epoch, __float_as_uint(ffn_act<KIND>(au + bu, ag + bgv)));
            }
        }
        return;
    }

    // ---------------- W_down (column tile, chunk)
    const int k = blockIdx.x - NU;
    const int tile = k % T, chunk = k / T;
    // Chunks in use: as many as give every row group at most one batch of
    // rows (the launch has G, the most).  Fewer, fuller chunks stream better,
    // and a second, mostly empty batch would cost as much as a full one.
    const int Ge = min(G, max(1, (nl + kSChunkRows - 1) / kSChunkRows));
    if (chunk >= Ge) return;
    // skip > 0: the hot prefix's FFN ran in the predictor's kernel, which has
    // ended.  Its epoch slots (read by nothing in this launch) advance here, by
    // tile 0's chunk 0 (present for every count): requested now, stored once
    // the chunk's rows are done, off the rows' path.
    const bool hot_slots = hT > 0 && k == 0;   // workgroup-uniform
    const uint32_t hsv = (hot_slots ? hslots : slots)[min(lane, (hot_slots ? hT : T) - 1)];   // no branch around it
    // skip > 0: chunk 0 of each tile adds the prefix's hG chunk partials (in
    // chunk order) for the tile's columns into the partial slot the last chunk
    // reads after the G others, once its rows are done (requested at the start,
    // the 24 values held across the rows made the OPT-30B-shaped step slower)
    const bool hot_sum = hG > 0 && chunk == 0;   // workgroup-uniform
    const int PD = (nl + Ge - 1) / Ge;
    const int j0 = sk + min(nl, chunk * PD), j1 = min(cnt, j0 + PD);
    const int ct = tid % kSColThreads;
    const int rg = __builtin_amdgcn_readfirstlane(tid / kSColThreads);
    const int col = tile * kFusedCols + ct * 8;
    const bool on = col < d;
    const int colc = min(col, d - 8);   // load address of a column past the end
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
    bool ok = true;
    uint32_t slot = 0;
    uint32_t epoch = 0;   // set with the first window (an empty chunk sets it after the loop)
    for (int w0 = j0; w0 < j1; w0 += kSWindow) {
        const int wn = min(kSWindow, j1 - w0);
        {
            int32_t v[kSWindow / kSThreads];
#pragma unroll
            for (int e = 0; e < kSWindow / kSThreads; ++e) v[e] = idx[w0 + min(tid + e * kSThreads, wn - 1)];
            slot = slots[min(lane, T - 1)];   // with the ids, after them
#pragma unroll
            for (int e = 0; e < kSWindow / kSThreads; ++e)
                if (tid + e * kSThreads < wn) s_row[tid + e * kSThreads] = min(max(v[e], 0), ffn - 1);
        }
        __syncthreads();
        const int nk = (wn - rg + kSGroups - 1) / kSGroups;   // this group's rows: rg + kSGroups * n
        // The first batch of rows goes out before the activations are collected
        // (overlapping the up rows they depend on).  A row whose activation
        // turns out to be 0 is still read: skipping it would have to wait for
        // the activation first, which costs more than the bytes it saves.
        u32x4 w[kSBatch];
        uint32_t wq[kSBatch];   // INT4: the row's code word and scale for the thread's 8 columns
        float wsc[kSBatch];
        auto load_row = [&](int q, int r) {
            if constexpr (Q4) {
                wq[q] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(
                    reinterpret_cast<const uint8_t*>(Wd) + (size_t)r * (d / 2) + colc / 2));
                wsc[q] = (float)sd[(size_t)r * (d >> 6) + (colc >> 6)];
            } else {
                w[q] = ld16_stream(Wd + (size_t)r * d + colc);
            }
        };
#pragma unroll
        for (int q = 0; q < kSBatch; ++q) load_row(q, s_row[min(rg + kSGroups * q, wn - 1)]);
        {
            uint64_t v[kSWindow / kSThreads];
#pragma unroll
            for (int e = 0; e < kSWindow / kSThreads; ++e) v[e] = ld_tag(&atag[w0 + min(tid + e * kSThreads, wn - 1)]);
            epoch = next_epoch(oldest_slot(slot));   // the slot load is long done by now
#pragma unroll
            for (int e = 0; e < kSWindow / kSThreads; ++e) {
                const int q = tid + e * kSThreads;
                if (q < wn) {
                    ok = poll_tag(&atag[w0 + q], v[e], epoch) && ok;
                    s_a[q] = __uint_as_float((uint32_t)v[e]);
                }
            }
        }
        __syncthreads();
        if (on) {
            for (int k0 = 0; k0 < nk; k0 += kSBatch) {
                if (k0 > 0) {
#pragma unroll
                    for (int q = 0; q < kSBatch; ++q) load_row(q, s_row[min(rg + kSGroups * (k0 + q), wn - 1)]);
                }
#pragma unroll
                for (int q = 0; q < kSBatch; ++q)
                    if (k0 + q < nk) {
                        if constexpr (Q4) axpy8_q4(acc, s_a[rg + kSGroups * (k0 + q)] * wsc[q], wq[q]);
                        else axpy8(acc, s_a[rg + kSGroups * (k0 + q)], w[q]);
                    }
            }
        }
        __syncthreads();
    }
    if (epoch == 0u) epoch = next_epoch(oldest_slot(slots[min(lane, T - 1)]));   // empty chunk (uniform)
    if (hot_slots && wave == 0) {
        const uint32_t he = next_epoch(oldest_slot(hsv));
        if (lane < hT) st_flag(&hslots[lane], he);
    }
    if (hot_sum && tile * kFusedCols + tid < d) {
        float hv[kHotMaxChunks];
        const int hc = tile * kFusedCols + tid;
#pragma unroll
        for (int g = 0; g < kHotMaxChunks; ++g) hv[g] = hpart[(size_t)min(g, hG - 1) * d + hc];
        float hs = 0.f;
#pragma unroll
        for (int g = 0; g < kHotMaxChunks; ++g)
            if (g < hG) hs += hv[g];
        st_coherent(&partial[(size_t)kFusedMaxChunks * d + tile * kFusedCols + tid], hs);
    }
    ok = __syncthreads_and(ok);
    *reinterpret_cast<f32x4*>(&s_red[rg][ct * 8]) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(&s_red[rg][ct * 8 + 4]) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    __syncthreads();
    // one column per thread: the chunk's partial (NaN if its activations never arrived)
    const int gc = tile * kFusedCols + tid;
    if (tid < kFusedCols && gc < d) {
        float v = 0.f;
#pragma unroll
        for (int g = 0; g < kSGroups; ++g) v += s_red[g][tid];
        st_coherent(&partial[(size_t)chunk * d + gc], ok ? v : __builtin_nanf(""));
    }
    wait_own_memory();
    __syncthreads();
    if (tid == 0) {
        uint32_t* c = &ctr[(size_t)tile * kCtrStride];
        const int flag = fetch_add(c, 1u) == (uint32_t)(Ge - 1);
        if (flag) st_flag(c, 0u);   // the last arrival puts the counter back for the next call
        s_flag = flag;
    }
    __syncthreads();
    if (!s_flag || tid >= kFusedCols || gc >= d) return;

    // the tile's last chunk: add the G partials in chunk order, all loads in one round
    // the partial buffer holds kFusedMaxChunks + 1 chunks, so every load is in bounds;
    // the last slot is the hot prefix's sum, stored by chunk 0
    float v[kFusedMaxChunks + 1];
#pragma unroll
    for (int g = 0; g < kFusedMaxChunks + 1; ++g) v[g] = ld_coherent(&partial[(size_t)g * d + gc]);
    float sum = 0.f;
#pragma unroll
    for (int g = 0; g < kFusedMaxChunks; ++g)
        if (g < Ge) sum += v[g];
    if (hG > 0) sum += v[kFusedMaxChunks];
    y[gc] = craw < 0 ? __builtin_nanf("") : sum;
    // every chunk of this tile has read the epoch: the tile's slot advances
    if (tid == 0) st_flag(&slots[tile], epoch);
}

// Hidden-row workgroups of a predict launch: none when every logits tile lies
// in the always-listed prefix.  The compaction (INT4: the last logits
// workgroup) stores the launch's epoch once it has every mask (count), and
// that orders the store after every other workgroup's read of the epoch only
// because a tile outside the prefix waits for every h; with no such tile a
// late hidden-row workgroup could read the stored epoch and publish h tagged
// as the next launch's, so none is launched.
static int hidden_workgroups(int r, int ffn, int hot) {
    const int NT = (ffn + kLTile - 1) / kLTile;
    return NT * kLTile <= hot ? 0 : (r + 3) / 4;
}

hipError_t launch_sparse_fused_q4(int kind, const h16* x, int d, int ffn, const uint8_t* qu, const h16* su,
                                  const float* bup, const uint8_t* qg, const h16* sg, const float* bg,
                                  const uint8_t* qd, const h16* sd, const int32_t* idx, const int32_t* count,
                                  float* y, const FusedSparseLayout& L, char* hdr, char* data, hipStream_t s) {
    uint64_t* atag = reinterpret_cast<uint64_t*>(data + L.atag);
    float* partial = reinterpret_cast<float*>(data + L.partial);
    uint32_t* ctr = reinterpret_cast<uint32_t*>(hdr + Sync::ffn_ctr);
    uint32_t* slots = reinterpret_cast<uint32_t*>(hdr + Sync::ffn_epoch);
    const float* zero = reinterpret_cast<const float*>(hdr + Sync::zero);
    const h16* wu = reinterpret_cast<const h16*>(qu);
    const h16* wg = reinterpret_cast<const h16*>(qg);
    const h16* wd = reinterpret_cast<const h16*>(qd);
    dim3 grid(L.NU + L.T * L.G);
#define PI_SFQ(K)                                                                                                    \
    hipLaunchKernelGGL((k_sparse_fused<K, true>), grid, dim3(kSThreads), 0, s, x, d, ffn, wu, bup, wg, bg, wd, idx, \
                       count, 0, L.NU, L.T, L.G, atag, partial, ctr, slots, y, zero, su, sg, sd)
    if (kind == 2) PI_SFQ(2);
    else if (kind == 1) PI_SFQ(1);
    else PI_SFQ(0);
#undef PI_SFQ
    return hipGetLastError();
}

hipError_t launch_predict_fused(const h16* x, int d, const h16* P1, const float* b1, bool relu, int r,
                                const h16* P2, const float* b2, int ffn, int hot, float thr,
                                const FusedPredLayout& L, char* hdr, char* data, int32_t* idx, int32_t* count,
                                hipStream_t s) {
    uint64_t* htag = reinterpret_cast<uint64_t*>(data + L.htag);
    uint64_t* desc = reinterpret_cast<uint64_t*>(data + L.desc);
    const int NA = hidden_workgroups(r, ffn, hot);
    const size_t shm = (size_t)(d * 2 > r * 4 ? d * 2 : r * 4);
    const float* zero = reinterpret_cast<const float*>(hdr + Sync::zero);
    hipLaunchKernelGGL((k_predict_fused<false, -1>), dim3(NA + L.NT + 1), dim3(256), shm, s, x, d, P1, b1, (int)relu,
                       r, P2, b2, ffn, thr, htag, desc, reinterpret_cast<uint32_t*>(hdr + Sync::pred_epoch), idx, count,
                       zero, hot, NA, nullptr, nullptr, HotArgs{});
    return hipGetLastError();
}

hipError_t launch_predict_fused_q4(const h16* x, int d, const uint8_t* q1, const h16* s1, const float* b1, bool relu,
                                   int r, const uint8_t* q2, const h16* s2, const float* b2, int ffn, int hot,
                                   float thr, const FusedPredLayout& L, char* hdr, char* data, int32_t* idx,
                                   int32_t* count, hipStream_t s) {
    uint64_t* htag = reinterpret_cast<uint64_t*>(data + L.htag);
    uint64_t* desc = reinterpret_cast<uint64_t*>(data + L.desc);
    const int NA = hidden_workgroups(r, ffn, hot);
    const size_t shm = (size_t)(d * 2 > r * 4 ? d * 2 : r * 4);
    const float* zero = reinterpret_cast<const float*>(hdr + Sync::zero);
    hipLaunchKernelGGL((k_predict_fused<true, -1>), dim3(NA + (L.NT + kQ4Tiles - 1) / kQ4Tiles), dim3(256), shm, s, x, d,
                       reinterpret_cast<const h16*>(q1), b1, (int)relu, r, reinterpret_cast<const h16*>(q2), b2, ffn,
                       thr, htag, desc, reinterpret_cast<uint32_t*>(hdr + Sync::pred_epoch), idx, count, zero, hot,
                       NA, s1, s2, HotArgs{});
    return hipGetLastError();
}

hipError_t launch_predict_fused_hot(int kind, const h16* x, int d, const h16* P1, const float* b1, bool relu, int r,
                                    const h16* P2, const float* b2, int ffn, int hot, float thr,
                                    const FusedPredLayout& L, char* hdr, char* data, int32_t* idx, int32_t* count,
                                    const h16* Wup, const float* bup, const h16* Wg, const float* bg, const h16* Wd,
                                    const HotLayout& HL, char* hot_area, hipStream_t s) {
    uint64_t* htag = reinterpret_cast<uint64_t*>(data + L.htag);
    uint64_t* desc = reinterpret_cast<uint64_t*>(data + L.desc);
    const int NA = hidden_workgroups(r, ffn, hot);
    // LDS: x (hidden rows; hot up rows, staged in whole 64-chunk blocks of 1 KB),
    // h (logits), the hot W_down row-group sums
    size_t shm = (size_t)((d * 2 + 1023) / 1024) * 1024;
    if (shm < (size_t)r * 4) shm = (size_t)r * 4;
    if (shm < (size_t)kHotGroups * kHotCols * 4) shm = (size_t)kHotGroups * kHotCols * 4;
    const float* zero = reinterpret_cast<const float*>(hdr + Sync::zero);
    HotArgs H{};
    H.Wu = Wup;
    H.bu = bup;
    H.Wg = Wg;
    H.bg = bg;
    H.Wd = Wd;
    H.atag = reinterpret_cast<uint64_t*>(hot_area + HL.atag);
    H.partial = reinterpret_cast<float*>(hot_area + HL.partial);
    H.slots = reinterpret_cast<uint32_t*>(hot_area + HL.slots);
    H.n = hot;
    H.NHU = hot > 0 ? ((hot + 3) / 4 < kHotUpMaxWG ? (hot + 3) / 4 : kHotUpMaxWG) : 0;
    H.G = hot > 0 ? hot_chunks(hot) : 0;
    H.T = HL.T;
    const dim3 grid(NA + H.NHU + L.NT + 1 + H.T * H.G);
#define PI_PH(K)                                                                                                    \
    hipLaunchKernelGGL((k_predict_fused<false, K>), grid, dim3(256), shm, s, x, d, P1, b1, (int)relu, r, P2, b2, ffn, \
                       thr, htag, desc, reinterpret_cast<uint32_t*>(hdr + Sync::pred_epoch), idx, count, zero, hot, NA, \
                       nullptr, nullptr, H)
    if (kind == 2) PI_PH(2);
    else if (kind == 1) PI_PH(1);
    else PI_PH(0);
#undef PI_PH
    return hipGetLastError();
}

hipError_t launch_sparse_fused(int kind, const h16* x, int d, int ffn, const h16* Wup, const float* bup,
                               const h16* Wg, const float* bg, const h16* Wd, const int32_t* idx,
                               const int32_t* count, float* y, const FusedSparseLayout& L, char* hdr,
                               char* data, hipStream_t s, int skip, const HotLayout* HL, char* hot_area) {
    uint64_t* atag = reinterpret_cast<uint64_t*>(data + L.atag);
    float* partial = reinterpret_cast<float*>(data + L.partial);
    uint32_t* ctr = reinterpret_cast<uint32_t*>(hdr + Sync::ffn_ctr);
    uint32_t* slots = reinterpret_cast<uint32_t*>(hdr + Sync::ffn_epoch);
    const float* zero = reinterpret_cast<const float*>(hdr + Sync::zero);
    const bool hot = skip > 0 && HL != nullptr;
    const float* hpart = hot ? reinterpret_cast<const float*>(hot_area + HL->partial) : nullptr;
    uint32_t* hslots = hot ? reinterpret_cast<uint32_t*>(hot_area + HL->slots) : nullptr;
    const int hG = hot ? hot_chunks(skip) : 0, hT = hot ? HL->T : 0;
    dim3 grid(L.NU + L.T * L.G);
#define PI_SF(K)                                                                                               \
    hipLaunchKernelGGL(k_sparse_fused<K>, grid, dim3(kSThreads), 0, s, x, d, ffn, Wup, bup, Wg, bg, Wd, idx, count, \
                       skip, L.NU, L.T, L.G, atag, partial, ctr, slots, y, zero, nullptr, nullptr, nullptr, hpart,   \
                       hG, hslots, hT)
    if (kind == 2) PI_SF(2);
    else if (kind == 1) PI_SF(1);
    else PI_SF(0);
#undef PI_SF
    return hipGetLastError();
}

// Zero n 32-bit words (a fill kernel, so that the call stays capturable in a graph).
__global__ __launch_bounds__(256) void k_zero(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    size_t g = (n + 255) / 256;
    if (g > 1024) g = 1024;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)g), dim3(256), 0, s, static_cast<uint32_t*>(p), n);
    return hipGetLastError();
}

}  // namespace pi
