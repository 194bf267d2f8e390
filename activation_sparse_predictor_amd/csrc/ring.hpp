// Skinny GEMM core of the batched path: R rows of one or two weight matrices
// (rows taken in list order, optionally through a row-id list) against up to
// 128 tokens, on the matrix cores, with both operands streamed through an LDS
// ring by direct-to-LDS loads.
//
// Load geometry.  One "block" is what a single wave-wide 16-byte-per-lane load
// moves: 8 rows x 128 contiguous bytes, written by global_load_lds_dwordx4 to
// 1 KB of LDS, lane j at bytes 16j: row j / 8, slot j % 8 of that row.  The
// eight lanes of a row cover its whole 128-byte line, so the load unit merges
// them; with lane j on row j % 8 instead (eight lines, one lane each per
// 16-byte step) the same loads ran at a third of the rate (measured on
// MI355X: 38 against 111 GB/s per CU from L2).  Chunk c of row r sits in slot
// c ^ blk_swz(r) = c ^ ((r / 2) % 8): the 16 lanes of one LDS read phase take
// rows r0 .. r0 + 15 at one chunk, and their 16-byte pieces land on 16
// different 4-bank groups (row parity picks the 128-byte half of the
// 256-byte bank cycle, the swizzle the 16-byte group in it).
//
// Stages.  A stage covers SEG 128-byte segments (64*SEG halves of K) of every
// operand row: NM matrices x RB rows and NX activation arrays x 8*XG tokens
// (the 8-token groups that hold a valid token; the matrix cores take tokens in
// blocks of 32, and the slots of a block past the loaded groups read a loaded
// group again: their sums are never used).
// The ring holds NS stages; stage s + NS - 1 is loaded while stage s is
// multiplied, and each wave waits only for its own loads of stage s (vmcnt),
// then a workgroup barrier makes every wave's loads visible.  Within a stage
// all of its LDS operand reads go out first and the MFMAs then run back to
// back; with at least two MFMAs per load, stage s + NS - 1's loads go out one
// at a time between them, else all at once after the barrier.
//
// MFMA.  v_mfma_f32_32x32x16_f16: lane l supplies row (or token) l % 32 and 8
// halves of K from chunk 2p + l / 32 of chunk pair p; the contraction order
// inside a stage is a permutation of K, the same for both operands.  Wave w
// takes token block w % NB and the chunk pairs p = w / NB (mod 4 / NB); with
// NB < 4 the waves that share a token block add their sums in LDS.  An fp32
// activation array is carried as two fp16 arrays (hi, lo) that add into the
// same accumulators (NX = 2).
//
// Work split (stream-K).  A unit is one stage of one RB-row block.  The
// T = row blocks x stages units are cut into gridDim.x equal ranges, one per
// workgroup, so every workgroup streams the same number of bytes whatever the
// row count (unless the row blocks fill at least 3/4 of the grid: then each
// workgroup takes one whole row block, see ring_gemm).  A row block whose stages all fall in one range is finished in
// place; otherwise each piece writes its fp32 sums to a slot of its own and
// the last piece to arrive on the row block's counter adds the pieces in
// workgroup order (fixed order: deterministic) and finishes the row block,
// then puts the counter back to 0.  When the rows are few and K is long (every
// row block split many ways), that one workgroup would read all the pieces
// alone: there the pieces are left for ring_finish, a kernel of their own
// that spreads the sums over the whole device.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace pi {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// Slot swizzle of the load blocks (see the load geometry above).
__host__ __device__ constexpr int blk_swz(int r) { return (r >> 1) & 7; }
// LDS byte offset, within a block, of chunk c of row r (the row's index in
// its row set, of which the block holds rows 8 * (r / 8) ..)
__device__ __forceinline__ int blk_off(int r, int c) { return ((r & 7) << 7) + ((c ^ blk_swz(r)) << 4); }
typedef float ring_f32x16 __attribute__((ext_vector_type(16)));

// Workgroup barrier without the memory fences of __syncthreads (those would
// make every wave wait for all of its outstanding loads, the ring's included);
// the empty asm keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// (dma16 and wait_vm, common.hpp: the ring's direct-to-LDS loads are issued
// as inline assembly, so that the compiler does not make every LDS read wait
// for all outstanding loads, which would drain the ring at every stage.)

template <int NM_, int NX_, int XG_, int RBW_, int SEG_, int NS_>
struct RingCfg {
    static constexpr int NM = NM_, NX = NX_, XG = XG_, RBW = RBW_, SEG = SEG_, NS = NS_;
    static constexpr int NB = (XG + 3) / 4;           // 32-token blocks
    static constexpr int RB = 32 * RBW;               // rows per row block
    static constexpr int BP = 32 * NB;                // token slots
    static constexpr int WBLK = NM * (RB / 8) * SEG;  // weight blocks per stage
    static constexpr int XBLK = NX * XG * SEG;        // activation blocks per stage
    static constexpr int NBLK = WBLK + XBLK;
    static constexpr int IPW = NBLK / 4;              // loads per wave per stage
    static constexpr int STAGE = NBLK * 1024;         // bytes per stage
    static constexpr int KST = SEG * 64;              // halves of K per stage
    static constexpr int WK = 4 / NB;                 // waves sharing a token block
    static constexpr int NPW = 4 * SEG / WK;          // chunk pairs per wave per stage
    static constexpr int NMF = NPW * RBW * NM * NX;   // MFMAs per wave per stage
    // per-wave sums: one block of 16 rows x 65 floats per (wave, row block of
    // 32, matrix), 1056 floats apart (see ring_gemm's epilogue)
    static constexpr int REDE = 65, REDB = 1056;
    static constexpr int RED = 4 * RBW * NM * REDB * 4;   // bytes of per-wave sums
    static constexpr int LDS = NS * STAGE > RED ? NS * STAGE : RED;
    static_assert(XG == 1 || XG == 2 || XG == 4 || XG == 8 || XG == 16, "token groups: 1, 2 or 4, or whole blocks");
    static_assert(WBLK % 4 == 0 && XBLK % 4 == 0 && IPW * (NS - 2) < 64, "loads per stage");
    static_assert(NS >= 2, "ring depth");
};

struct RingArgs {
    const h16* W[2];          // NM weight matrices, row stride ldw halves
    int ldw;
    const int32_t* rowlist;   // row ids of the list (gathering kernels only)
    int wrows;                // rows of W (a gathered id is clamped to them)
    int nrows;                // list length
    const h16* X[2];          // NX activation arrays [token][ldx]
    int ldx;
    int B;                    // valid tokens, at most 8*XG (loads of slots B.. read zeros)
    int K;                    // contraction length in halves (multiple of 8)
    const h16* zsrc;          // 16 zero bytes
    float* part;              // 2 * gridDim.x pieces of NM x BP x RB fp32 sums
    uint32_t* ctr;            // one arrival counter per row block, 0 between calls
};

// Runs the calling workgroup's range of units over the first nrows rows of
// the list (a.nrows is not read: a kernel may take the count from memory).
// GATHER: row i is a.rowlist[i], else row i.  LAST_FINISHES: a split row
// block is finished by the workgroup of its last piece (else by ring_finish,
// in a launch of its own).  The caller's LDS area lds holds C::LDS bytes,
// 16-byte aligned; the pieces area (a.part) holds two slots per workgroup of
// NM x BP x RB fp32 sums.
//
// The epilogue runs one row of a finished row block per thread (thread k:
// row k % RB, token slots k / RB + j * 256 / RB), so the 32 rows of a
// half-wave belong to one token.  epi.row(i) is called once per thread and
// row block and returns what the row's outputs need from memory (ids,
// biases); epi.apply<E>(i, row, t, v0, v1) then takes E token slots of that
// row at once, every thread uniformly, so that the loads of the E outputs go
// out together instead of one latency per output (at 128 tokens a thread
// holds 64 outputs of each row block).  v0 and v1 are the sums for matrices 0
// and 1 (v1 = 0 when NM = 1), 0 for t >= B; i runs to the end of the row
// block, past nrows, where the sums mean nothing.
template <class C, bool GATHER, bool LAST_FINISHES, class Epi>
__device__ __forceinline__ void ring_gemm(const RingArgs& a, int nrows, char* lds, Epi&& epi) {
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar block arithmetic
    const int li = lane & 31, kh = lane >> 5;
    const int wn = wave % C::NB, wk = wave / C::NB;
    const int nrb = (nrows + C::RB - 1) / C::RB;
    const int nst = (a.K + C::KST - 1) / C::KST;
    const long long T = (long long)nrb * nst;
    // no more workgroups than units, so that no range is empty and every
    // workgroup between the first and last holder of a row block has a piece.
    // When the row blocks fill at least 3/4 of the grid they are not split:
    // one whole row block per workgroup (up to a third more stages each,
    // against the split blocks at both ends of a workgroup's range, whose
    // pieces, arrivals and last-arriver reads cost ~20 us each at 128 tokens
    // against ~8 us for a block finished in place).  (Only where the last
    // piece finishes: ring_finish assumes the even split.)
    const int gd = (int)gridDim.x;
    const bool whole_blocks = LAST_FINISHES && nrb <= gd && 4 * nrb >= 3 * gd;
    const int G = whole_blocks ? nrb : (int)min((long long)gd, T), w = (int)blockIdx.x;
    if (w >= G) return;
    static_assert(256 % C::RB == 0, "a thread keeps one row of the block");
    constexpr int kTS = 256 / C::RB;                // token-slot stride of a thread
    constexpr int kNT = C::BP / kTS;                // token slots per thread
    constexpr int kE = kNT < 16 ? kNT : 16;         // outputs per epilogue batch
    static_assert(kNT % kE == 0, "whole batches");
    const long long ua = T * w / G, ub = T * (w + 1) / G;
    float* red = reinterpret_cast<float*>(lds);
    const uint32_t lbase = (uint32_t)(size_t)(lds_void_ptr)lds;

    for (long long u = ua; u < ub;) {
        const int rb = (int)(u / nst), st0 = (int)(u % nst);
        const int st1 = (int)min((long long)nst, st0 + (ub - u));
        u += st1 - st0;
        const int n = st1 - st0;

        // this thread's loads: block b = wave + 4i of every stage
        const h16* src[C::IPW];
        int kofs[C::IPW];
        bool ok[C::IPW];
        // (WBLK is a multiple of 4, so block wave + 4i is a weight block
        // exactly when i < WBLK / 4, whatever the wave: no branches, and all
        // the row ids are in flight together)
#pragma unroll
        for (int i = 0; i < C::IPW; ++i) {
            const int b = wave + 4 * i;
            if (i < C::WBLK / 4) {
                const int m = b / ((C::RB / 8) * C::SEG), rem = b % ((C::RB / 8) * C::SEG);
                const int g = rem / C::SEG, sg = rem % C::SEG;
                const int rlr = g * 8 + (lane >> 3);   // the lane's row within the row block
                const int row = min(rb * C::RB + rlr, nrows - 1);
                const int id = GATHER ? min(max(a.rowlist[row], 0), a.wrows - 1) : row;
                src[i] = (m == 0 ? a.W[0] : a.W[1]) + (size_t)id * a.ldw;
                kofs[i] = sg * 64 + (((lane & 7) ^ blk_swz(rlr)) << 3);
                ok[i] = true;
            } else {
                const int bx = b - C::WBLK;
                const int ix = bx / (C::XG * C::SEG), rem = bx % (C::XG * C::SEG);
                const int tg = rem / C::SEG, sg = rem % C::SEG;
                const int t = tg * 8 + (lane >> 3);
                src[i] = (ix == 0 ? a.X[0] : a.X[1]) + (size_t)min(t, a.B - 1) * a.ldx;
                kofs[i] = sg * 64 + (((lane & 7) ^ blk_swz(t)) << 3);
                ok[i] = t < a.B;
            }
        }
        auto issue1 = [&](int st, int q, int i) {
            const uint32_t dst = lbase + q * C::STAGE;
            const int k = st * C::KST + kofs[i];
            const h16* p = (ok[i] && k < a.K) ? src[i] + k : a.zsrc;
            if (i < C::WBLK / 4) dma16_stream(p, dst + (wave + 4 * i) * 1024);   // weights: read once
            else dma16(p, dst + (wave + 4 * i) * 1024);
        };
        auto issue = [&](int st, int q) {
#pragma unroll
            for (int i = 0; i < C::IPW; ++i) issue1(st, q, i);
        };

        ring_f32x16 acc[C::RBW][C::NM];
#pragma unroll
        for (int rr = 0; rr < C::RBW; ++rr)
#pragma unroll
            for (int m = 0; m < C::NM; ++m) acc[rr][m] = ring_f32x16{};

        wait_vm<0>();   // nothing else outstanding: the ring waits count this unit's loads only
#pragma unroll
        for (int j = 0; j < C::NS - 1; ++j)
            if (j < n) issue(st0 + j, j);
        // stage s; MORE: a stage s + NS - 1 exists.  All of the stage's LDS
        // reads go out first, so that its MFMAs then run back to back instead
        // of each waiting for its read.  With at least two MFMAs per load the
        // next stage's loads go out between the MFMAs: a load instruction
        // holds its wave while the load unit takes its 1 KB, and the MFMAs
        // issued before it run on meanwhile (issued all together, the loads
        // and the MFMAs took turns).  With fewer, the loads go out at once,
        // as early as the ring allows.
        constexpr bool kSpread = C::NMF >= 2 * C::IPW;
        auto stage = [&](int s, auto MORE) {
            if (s + C::NS - 2 < n) wait_vm<(C::NS - 2) * C::IPW>();
            else wait_vm<0>();
            ring_barrier();   // stage s is in LDS; every wave is done with stage s - 1
            const int sn = st0 + s + C::NS - 1, qn = (s + C::NS - 1) % C::NS;
            if constexpr (decltype(MORE)::value && !kSpread) issue(sn, qn);
            const char* buf = lds + (s % C::NS) * C::STAGE;
            f16x8 xv[C::NPW][C::NX], wv[C::NPW][C::RBW][C::NM];
#pragma unroll
            for (int j = 0; j < C::NPW; ++j) {
                const int p = wk + j * C::WK;
                const int c = 2 * p + kh, sg = c >> 3, cc = c & 7;
                const int t = wn * 32 + li, tg = min(t >> 3, C::XG - 1);
#pragma unroll
                for (int ix = 0; ix < C::NX; ++ix) {
                    const int blk = C::WBLK + (ix * C::XG + tg) * C::SEG + sg;
                    xv[j][ix] = *reinterpret_cast<const f16x8*>(buf + blk * 1024 + blk_off(tg * 8 + (t & 7), cc));
                }
#pragma unroll
                for (int rr = 0; rr < C::RBW; ++rr) {
                    const int rl = rr * 32 + li, g = rl >> 3;
#pragma unroll
                    for (int m = 0; m < C::NM; ++m) {
                        const int blk = (m * (C::RB / 8) + g) * C::SEG + sg;
                        wv[j][rr][m] = *reinterpret_cast<const f16x8*>(buf + blk * 1024 + blk_off(rl, cc));
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < C::NPW; ++j)
#pragma unroll
                for (int rr = 0; rr < C::RBW; ++rr)
#pragma unroll
                    for (int m = 0; m < C::NM; ++m)
#pragma unroll
                        for (int ix = 0; ix < C::NX; ++ix) {
                            const int f = ((j * C::RBW + rr) * C::NM + m) * C::NX + ix;
                            if constexpr (decltype(MORE)::value && kSpread) {
#pragma unroll
                                for (int i = 0; i < C::IPW; ++i)
                                    if (i * C::NMF / C::IPW == f) issue1(sn, qn, i);
                            }
                            acc[rr][m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(wv[j][rr][m], xv[j][ix], acc[rr][m], 0, 0, 0);
                            __builtin_amdgcn_sched_barrier(0);
                        }
        };
        int s = 0;
        for (; s + C::NS - 1 < n; ++s) stage(s, std::true_type{});
        for (; s < n; ++s) stage(s, std::false_type{});
        ring_barrier();   // the ring is no longer read: its memory holds the sums now
#pragma unroll
        for (int rr = 0; rr < C::RBW; ++rr)
#pragma unroll
            for (int m = 0; m < C::NM; ++m)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    red[((wave * C::RBW + rr) * C::NM + m) * C::REDB + e * C::REDE + ((rr & 1) << 4) + lane] = acc[rr][m][e];
        __syncthreads();
        // sum of row rl, token slot t, matrix m: output (r, n) of a 32 x 32
        // block is element (r/8)*4 + r%4 of lane n + 32*((r/4)%2).  The
        // epilogue reads 64 rows of one token per wave instruction: the
        // element rows 65 floats apart and the odd row blocks shifted by 16
        // put those 64 reads on 64 different banks (unpadded, the 32 rows of
        // a row block would all hit one bank).  The blocks of the waves that
        // split K are added in wave order.
        auto val = [&](int m, int rl, int t) {
            const int rr = rl >> 5, r = rl & 31, tb = t >> 5, nn = t & 31;
            const int e = ((r >> 3) << 2) + (r & 3), ln = nn + (((r >> 2) & 1) << 5);
            float v = 0.f;
#pragma unroll
            for (int k = 0; k < C::WK; ++k)
                v += red[(((k * C::NB + tb) * C::RBW + rr) * C::NM + m) * C::REDB + e * C::REDE + ((rr & 1) << 4) + ln];
            return v;
        };
        // this thread's row and token slots: rl, tt + j * TS for j < NT (made
        // opaque in every unit: hoisted out of the unit loop, the epilogue's
        // addresses stayed live across the whole loop and were spilled)
        int rl = tid % C::RB, tt = tid / C::RB;
        asm volatile("" : "+v"(rl), "+v"(tt));
        const int row = rb * C::RB + rl;
        const bool whole = st0 == 0 && st1 == nst;
        // piece slot: kind 0 when the range starts inside this row block
        // (its first piece), 1 when it ends inside it (its last piece)
        auto slot = [&](int wg) {
            const int kind = (T * wg / G) >= (long long)rb * nst ? 0 : 1;
            return a.part + (size_t)(wg * 2 + kind) * C::NM * C::BP * C::RB;
        };
        // token slots j0 .. j1 - 1 of the sums in LDS: outputs of a whole row
        // block, or this workgroup's piece of a split one
        auto emit = [&](int j0, int j1, const auto& pr) {
            if (whole) {
                for (int j = j0; j < j1; j += kE) {
                    int t[kE];
                    float v0[kE], v1[kE];
#pragma unroll
                    for (int k = 0; k < kE; ++k) {
                        t[k] = tt + (j + k) * kTS;
                        v0[k] = val(0, rl, t[k]);
                        v1[k] = C::NM > 1 ? val(C::NM - 1, rl, t[k]) : 0.f;
                    }
                    epi.template apply<kE>(row, pr, t, v0, v1);
                }
            } else {
                float* mine = slot(w);
                for (int j = j0; j < j1; ++j) {
                    const int t = tt + j * kTS;
                    if (t < a.B && row < nrows)
#pragma unroll
                        for (int m = 0; m < C::NM; ++m) {
                            if (LAST_FINISHES) st_coherent(&mine[(m * C::BP + t) * C::RB + rl], val(m, rl, t));
                            else mine[(m * C::BP + t) * C::RB + rl] = val(m, rl, t);
                        }
                }
            }
        };
        emit(0, kNT, epi.row(row));
        if (!whole) {
            if (!LAST_FINISHES) {
                __syncthreads();   // the sums are read: the ring may be loaded again
                continue;
            }
            wait_own_memory();
            __syncthreads();
            // workgroups holding units rb*nst and (rb+1)*nst - 1
            const int wf = (int)((((long long)rb * nst + 1) * G + T - 1) / T) - 1;
            const int wl = (int)((((long long)(rb + 1) * nst) * G + T - 1) / T) - 1;
            if (tid == 0) {
                const bool last = fetch_add(&a.ctr[rb], 1u) == (uint32_t)(wl - wf);
                if (last) st_flag(&a.ctr[rb], 0u);
                s_last = last;
            }
            __syncthreads();
            if (s_last) {
                const auto pr = epi.row(row);
                for (int j = 0; j < kNT; j += kE) {
                    int t[kE];
                    float v0[kE], v1[kE];
#pragma unroll
                    for (int k = 0; k < kE; ++k) {
                        t[k] = tt + (j + k) * kTS;
                        v0[k] = 0.f;
                        v1[k] = 0.f;
                    }
                    for (int w0 = wf; w0 <= wl; ++w0) {   // pieces in order, kE outputs' loads in flight
                        const float* pc = slot(w0);
                        float x0[kE], x1[kE];
                        // (unconditional loads inside the slot, masked after:
                        // loads under a branch would cost a full wait each)
#pragma unroll
                        for (int k = 0; k < kE; ++k) {
                            x0[k] = ld_coherent(&pc[t[k] * C::RB + rl]);
                            x1[k] = C::NM > 1 ? ld_coherent(&pc[(C::BP + t[k]) * C::RB + rl]) : 0.f;
                        }
#pragma unroll
                        for (int k = 0; k < kE; ++k) {
                            const bool ok = t[k] < a.B && row < nrows;
                            v0[k] += ok ? x0[k] : 0.f;
                            v1[k] += ok ? x1[k] : 0.f;
                        }
                    }
                    epi.template apply<kE>(row, pr, t, v0, v1);
                }
            }
        }
        __syncthreads();   // the sums are read: the ring may be loaded again
    }
}

// Finishes the row blocks that a ring_gemm<C, ..., false> launch of G0
// workgroups left in pieces: one thread per (row block, token < B, row),
// grid-stride; each sums its pieces in workgroup order, 8 loads in flight.
// A thread finds its workgroup range once: only its first piece can be the
// second (tail) slot of its workgroup, every later workgroup starts inside
// the row block.  (Per-piece 64-bit divisions had made this kernel
// instruction-bound.)
template <class C, class Epi>
__device__ __forceinline__ void ring_finish(const RingArgs& a, int nrows, int G0, Epi&& epi) {
    const int nrb = (nrows + C::RB - 1) / C::RB;
    const int nst = (a.K + C::KST - 1) / C::KST;
    const long long T = (long long)nrb * nst;
    if (T == 0) return;
    const int G = (int)min((long long)G0, T);
    const bool narrow = T * (G + 1) < (1ll << 32);   // the unit arithmetic fits 32 bits
    const int BR = a.B * C::RB;   // outputs per row block
    const int total = nrb * BR;
    constexpr size_t kSlot = (size_t)C::NM * C::BP * C::RB;
    constexpr int kBatch = 8;   // pieces in flight (16 measured no faster)
    for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += gridDim.x * blockDim.x) {
        const int rb = e / BR, rem = e - rb * BR;
        const int t = rem / C::RB, rl = rem % C::RB;
        // workgroups wf .. wl hold the row block's units u0 .. u0 + nst - 1;
        // kf: workgroup wf's slot for it (1 when its range starts earlier)
        int wf, wl, kf;
        if (narrow) {
            const uint32_t u0 = (uint32_t)(rb * nst), Tu = (uint32_t)T, Gu = (uint32_t)G;
            wf = (int)(((u0 + 1) * Gu + Tu - 1) / Tu) - 1;
            wl = (int)(((u0 + nst) * Gu + Tu - 1) / Tu) - 1;
            kf = Tu * (uint32_t)wf / Gu >= u0 ? 0 : 1;
        } else {
            const long long u0 = (long long)rb * nst;
            wf = (int)(((u0 + 1) * G + T - 1) / T) - 1;
            wl = (int)(((u0 + nst) * G + T - 1) / T) - 1;
            kf = T * wf / G >= u0 ? 0 : 1;
        }
        if (wf == wl || rb * C::RB + rl >= nrows) continue;   // finished in place, or past the rows
        const float* p0 = a.part + (size_t)(t * C::RB + rl);
        const float* p1 = p0 + (size_t)(C::NM - 1) * C::BP * C::RB;
        float v0 = 0.f, v1 = 0.f;
        for (int w0 = wf; w0 <= wl; w0 += kBatch) {
            float x0[kBatch], x1[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int wg = min(w0 + j, wl);
                const size_t off = (size_t)(wg * 2 + (wg == wf ? kf : 0)) * kSlot;
                x0[j] = p0[off];
                x1[j] = C::NM > 1 ? p1[off] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                if (w0 + j <= wl) {
                    v0 += x0[j];
                    v1 += x1[j];
                }
        }
        const int i = rb * C::RB + rl;
        const int tt[1] = {t};
        const float a0[1] = {v0}, a1[1] = {v1};
        epi.template apply<1>(i, epi.row(i), tt, a0, a1);
    }
}

}  // namespace pi
