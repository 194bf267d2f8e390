// Internal launch interface and workspace layout of the sparse-FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pi {

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---- predictor: logits tiles of 64 neurons (one wave-wide ballot each).
// Tiles arrive on a two-level counter: level 1 has kArriveGroups counters
// (tile % kArriveGroups), level 2 one counter; each sits on its own 128-byte
// line so arrivals on different counters do not serialize.
constexpr int kPredTile = 64;
constexpr int kArriveGroups = 8;
constexpr int kCtrStride = 32;   // uint32 words between counters (128 bytes)
constexpr int kCtrWords = (kArriveGroups + 1) * kCtrStride;   // per token
__host__ __device__ inline int pred_tiles(int ffn) { return (ffn + kPredTile - 1) / kPredTile; }

// ---- W_down accumulate: column tiles of 1024 (128 threads x 8 fp16), each
// workgroup split into kDownGroups row groups reduced in LDS, and G neuron
// chunks per tile combined in a fixed order (deterministic).
constexpr int kDownColThreads = 128;
constexpr int kDownGroups = 8;
constexpr int kDownThreads = kDownColThreads * kDownGroups;
constexpr int kDownCols = kDownColThreads * 8;
constexpr int kDownMaxChunks = 64;
constexpr int kDownWindow = kDownThreads;   // active-list entries staged in LDS at a time
inline int down_tiles(int d) { return (d + kDownCols - 1) / kDownCols; }
inline int down_chunks(int d, int ffn) {
    int T = down_tiles(d);
    int G = 256 / T;   // at most one workgroup per CU in flight
    if (G < 1) G = 1;
    if (G > kDownMaxChunks) G = kDownMaxChunks;
    if (G > ffn) G = ffn;
    return G;
}

struct SparseLayout {
    size_t a;        // B x ffn fp32 activations, in active-list order
    size_t partial;  // B x G x d fp32 per-chunk partial outputs
    size_t ctr;      // B x T arrival counters, kCtrStride words apart
    size_t total;
    int T, G;
};

inline SparseLayout sparse_layout(int B, int d, int ffn) {
    SparseLayout L;
    L.T = down_tiles(d);
    L.G = down_chunks(d, ffn);
    L.a = 0;
    L.partial = align256((size_t)B * ffn * 4);
    L.ctr = L.partial + align256((size_t)B * L.G * d * 4);
    L.total = L.ctr + align256((size_t)B * L.T * kCtrStride * 4);
    return L;
}

// ---- batched union path (2 <= B <= kUnionMaxTokens tokens per pass)
constexpr int kUnionMaxTokens = 128;
// Skinny GEMMs of the batched path (ring.hpp): at most kRingMaxWG workgroups,
// token slots padded to 32, 64 or 128 and row blocks of as many rows.  Piece
// area: two slots per workgroup of (matrices x token slots x rows) fp32 sums.
constexpr int kRingMaxWG = 1024;
constexpr int kRingRows = 32;
inline int ring_slots(int B) { return B <= 32 ? 32 : (B <= 64 ? 64 : 128); }
// 8-token groups loaded for B tokens, and 32-row blocks per row block for xg
// groups, by kernel: the row block grows with the tokens, to keep the
// activation bytes per weight byte of a stage down (the logits read h as two
// arrays, hi and lo, so theirs grows first; the hidden layer has few rows, so
// its stays small: a larger one would split each row block more ways)
__host__ __device__ constexpr int ring_xg(int B) {
    return B <= 8 ? 1 : (B <= 16 ? 2 : (B <= 32 ? 4 : (B <= 64 ? 8 : 16)));
}
__host__ __device__ constexpr int rbw_up(int xg) { return xg <= 2 ? 1 : (xg == 4 ? 2 : xg / 4); }
__host__ __device__ constexpr int rbw_hidden(int xg) { return xg <= 4 ? 1 : 2; }
__host__ __device__ constexpr int rbw_logits(int xg) { return xg <= 4 ? xg : 4; }
inline size_t ring_piece_bytes(int nm, int rbw, int B) {
    return (size_t)2 * kRingMaxWG * nm * ring_slots(B) * (32 * rbw) * 4;
}
struct BatchLayout {
    size_t tokbits;  // B x ceil(ffn/32) uint32 per-token bitmaps of the lists
    size_t umasks;   // tiles uint64 union bitmaps
    size_t ulist;    // ffn int32 ascending union list
    size_t ucount;   // uint32 |U|
    size_t aT;       // Bp x lda fp16 activations, token-major
    size_t partial;  // G x Bp x d fp32 chunk partials of the down GEMM
    size_t ctr;      // kCtrWords uint32 arrival counters
    size_t upctr;    // ceil(ffn/64) uint32 row-block counters of the up GEMM
    size_t upart;    // pieces of the up GEMM (two matrices for ReGLU)
    size_t total;
    int W, Bp, lda, G;
};

// Union chunks of the down GEMM for B tokens (batch.hip): its grid is
// (column tiles, chunks), and the chunk count is picked to fill whole waves
// of the device (1 to 64 chunks; the partials are chunks x Bp x d).
int union_down_chunks(int B, int d);

inline BatchLayout batch_layout(int B, int d, int ffn) {
    BatchLayout L;
    L.W = (B + 31) / 32;
    L.Bp = L.W * 32;
    L.lda = (ffn + 7) & ~7;
    L.G = union_down_chunks(B, d);
    const size_t tiles = (size_t)(ffn + 63) / 64;
    L.tokbits = 0;
    L.umasks = L.tokbits + align256((size_t)B * ((ffn + 31) / 32) * 4);
    L.ulist = L.umasks + align256(tiles * 8);
    L.ucount = L.ulist + align256((size_t)ffn * 4);
    L.aT = L.ucount + 256;
    L.partial = L.aT + align256((size_t)L.Bp * L.lda * 2);
    L.ctr = L.partial + align256((size_t)L.G * L.Bp * d * 4);
    L.upctr = L.ctr + align256((size_t)kCtrWords * 4);
    L.upart = L.upctr + align256((size_t)((ffn + kRingRows - 1) / kRingRows) * 4);
    L.total = L.upart + align256(ring_piece_bytes(2, rbw_up(ring_xg(B)), B));
    return L;
}

// ---- batched predictor (2 <= B <= kUnionMaxTokens tokens per pass)
struct BPredLayout {
    size_t h_hi, h_lo;   // Bp x ldh fp16 hidden activations (hi + lo)
    size_t masks32;      // B x ceil(ffn/32) uint32 per-token tile masks
    size_t hpart;        // pieces of the hidden and logits GEMMs (one after the other)
    size_t lctr;         // ceil(ffn/64) uint32 row-block counters of the logits GEMM
    size_t total;
    int Bp, ldh;
};

inline BPredLayout bpred_layout(int B, int r, int ffn) {
    BPredLayout L;
    L.Bp = ((B + 31) / 32) * 32;
    L.ldh = (r + 7) & ~7;
    L.h_hi = 0;
    L.h_lo = align256((size_t)L.Bp * L.ldh * 2);
    L.masks32 = L.h_lo + align256((size_t)L.Bp * L.ldh * 2);
    L.hpart = L.masks32 + align256((size_t)B * ((ffn + 31) / 32) * 4);
    const int rbw = rbw_hidden(ring_xg(B)) > rbw_logits(ring_xg(B)) ? rbw_hidden(ring_xg(B)) : rbw_logits(ring_xg(B));
    L.lctr = L.hpart + align256(ring_piece_bytes(1, rbw, B));
    L.total = L.lctr + align256((size_t)((ffn + kRingRows - 1) / kRingRows) * 4);
    (void)r;
    return L;
}

// ---- fused single-token kernels.  They publish intermediate values as
// tagged 64-bit words {launch epoch, payload} in the data area, and keep
// their epochs and the W_down arrival counters in a fixed header at the start
// of every workspace, which no other layout touches: the header is zero-filled
// once when the workspace is allocated; each counter is put back to 0 by the
// last arrival of every call, and each epoch advances by one per launch on
// the device (so a captured graph replays with a new epoch each time).  A
// call's data area starts kSyncBytes in (pi_ffn_decode puts the FFN's data
// area after the predictor's, behind the one header they share: predict and
// the FFN use disjoint header fields).
constexpr int kFusedCols = 512;                     // W_down columns per tile
constexpr int kFusedMaxTiles = 16384 / kFusedCols;  // PI_MAX_D / kFusedCols
constexpr int kFusedMaxChunks = 48;                 // list chunks per W_down tile
struct Sync {   // byte offsets inside the header
    static constexpr size_t ffn_ctr = 0;                                    // one line per W_down tile
    static constexpr size_t ffn_epoch = ffn_ctr + (size_t)kFusedMaxTiles * kCtrStride * 4;  // per tile
    static constexpr size_t pred_epoch = ffn_epoch + kFusedMaxTiles * 4;    // last predict launch's epoch
    static constexpr size_t zero = pred_epoch + 128;                        // never written
    static constexpr size_t end = zero + 256;
};
constexpr size_t kSyncBytes = 8192;
static_assert(Sync::end <= kSyncBytes, "sync header overflow");

struct FusedPredLayout {
    size_t htag, desc, total;   // offsets from the data area; the whole layout is tagged words
    int NT;
};
inline FusedPredLayout fused_pred_layout(int r, int ffn) {
    FusedPredLayout L;
    L.NT = (ffn + 31) / 32;
    L.htag = 0;   // padded to a multiple of 1024 words: the collection reads whole rounds
    // the fp16 predictor's tile masks (8 bytes a tile), or the INT4
    // predictor's look-back descriptors (128 bytes per four tiles)
    L.desc = align256((size_t)((r + 1023) / 1024) * 1024 * 8);
    L.total = L.desc + align256((size_t)(L.NT + 3) / 4 * 128);
    return L;
}

struct FusedSparseLayout {
    size_t atag, partial, total;   // offsets from the data area; [atag, partial) is tagged words
    int NU, T, G;
};
inline FusedSparseLayout fused_sparse_layout(int d, int ffn) {
    FusedSparseLayout L;
    L.T = (d + kFusedCols - 1) / kFusedCols;
    L.G = kFusedMaxChunks;   // launched; the kernel uses as many as the count needs
    if (L.G > ffn) L.G = ffn;
    if (L.G < 1) L.G = 1;
    L.NU = (ffn + 7) / 8 < 384 ? (ffn + 7) / 8 : 384;   // up chunks (8 waves each)
    L.atag = 0;
    L.partial = align256((size_t)ffn * 8);
    // padded: the reduction reads every chunk slot, and one more, kFusedMaxChunks,
    // which holds the hot prefix's sum (chunk 0 adds the predictor's kernel's
    // chunk partials into it)
    L.total = L.partial + align256((size_t)(kFusedMaxChunks + 1) * d * 4);
    return L;
}

// ---- the always-listed hot prefix's FFN inside the predictor's kernel
// (pi_ffn_decode_hot, B = 1).  Its own area of the decode workspace, behind
// the predictor's data area: the W_down tiles' epoch slots, the prefix's
// activations as tagged words, and the chunk partials, which the FFN kernel
// that follows adds to y.  Zero-filled with the other tagged words whenever
// the workspace held another layout; after that the slots advance by one per
// step (in the FFN kernel, once the predictor's kernel has ended).
constexpr int kHotRowsPerChunk = 64;   // 4 row groups x 16 rows in flight
constexpr int kHotMaxChunks = 24;   // the FFN's last chunk of a tile reads 24 of them in its round
struct HotLayout {
    size_t slots, atag, partial, total;   // offsets from the hot area's start
    int T;
};
inline HotLayout hot_layout(int d, int ffn) {
    HotLayout L;
    L.T = (d + kFusedCols - 1) / kFusedCols;
    L.slots = 0;
    L.atag = L.slots + 256;
    L.partial = L.atag + align256((size_t)ffn * 8);
    L.total = L.partial + align256((size_t)kHotMaxChunks * d * 4);
    return L;
}
// chunks of the prefix per W_down column tile: whole 64-row batches, at most kHotMaxChunks
inline int hot_chunks(int n) {
    const int g = (n + kHotRowsPerChunk - 1) / kHotRowsPerChunk;
    return g < kHotMaxChunks ? g : kHotMaxChunks;
}

typedef _Float16 h16;

// sparse.hip
hipError_t launch_up_act(int kind, bool dense, const h16* x, int B, int d, int ffn,
                         const h16* Wup, const float* bup, const h16* Wg, const float* bg,
                         const int32_t* idx, const int32_t* count, float* a, uint32_t* ctr,
                         int T, hipStream_t s);
hipError_t launch_down_acc(bool dense, const h16* Wd, int B, int d, int ffn, const int32_t* idx,
                           const int32_t* count, const float* a, float* y, float* partial,
                           uint32_t* ctr, int T, int G, hipStream_t s);

// batch.hip
hipError_t launch_union(int kind, const h16* x, int B, int d, int ffn, const h16* Wup,
                        const float* bup, const h16* Wg, const float* bg, const h16* Wd,
                        const int32_t* idx, const int32_t* count, float* y, const BatchLayout& L,
                        char* ws, char* hdr, hipStream_t s);

hipError_t launch_check_idx(const int32_t* idx, const int32_t* count, int B, int ffn, int d, float* y,
                            hipStream_t s);

hipError_t launch_bpredict(const h16* x, int B, int d, const h16* P1, const float* b1, bool relu,
                          const h16* P2, const float* b2, int r, int ffn, int hot, float thr, int32_t* idx,
                          int32_t* count, const BPredLayout& L, char* ws, char* hdr, hipStream_t s);

// fused.hip
hipError_t launch_predict_fused(const h16* x, int d, const h16* P1, const float* b1, bool relu, int r,
                                const h16* P2, const float* b2, int ffn, int hot, float thr,
                                const FusedPredLayout& L, char* hdr, char* data, int32_t* idx, int32_t* count,
                                hipStream_t s);
// The same launch with the hot prefix's FFN ([0, hot) rows of W_up [W_gate]
// W_down) computed in the kernel's extra roles: its chunk partials stay in the
// hot area, and the following launch_sparse_fused(..., skip = hot) adds them
// to y and advances the hot area's epoch slots.
hipError_t launch_predict_fused_hot(int kind, const h16* x, int d, const h16* P1, const float* b1, bool relu, int r,
                                    const h16* P2, const float* b2, int ffn, int hot, float thr,
                                    const FusedPredLayout& L, char* hdr, char* data, int32_t* idx, int32_t* count,
                                    const h16* Wup, const float* bup, const h16* Wg, const float* bg, const h16* Wd,
                                    const HotLayout& HL, char* hot_area, hipStream_t s);
hipError_t launch_predict_fused_q4(const h16* x, int d, const uint8_t* q1, const h16* s1, const float* b1, bool relu,
                                   int r, const uint8_t* q2, const h16* s2, const float* b2, int ffn, int hot,
                                   float thr, const FusedPredLayout& L, char* hdr, char* data, int32_t* idx,
                                   int32_t* count, hipStream_t s);
// skip > 0: list positions [0, skip) (the hot prefix) were computed by
// launch_predict_fused_hot, whose chunk partials (in hot_area, laid out by HL)
// are added to y.
hipError_t launch_sparse_fused(int kind, const h16* x, int d, int ffn, const h16* Wup, const float* bup,
                               const h16* Wg, const float* bg, const h16* Wd, const int32_t* idx,
                               const int32_t* count, float* y, const FusedSparseLayout& L, char* hdr,
                               char* data, hipStream_t s, int skip = 0, const HotLayout* HL = nullptr,
                               char* hot_area = nullptr);
hipError_t launch_sparse_fused_q4(int kind, const h16* x, int d, int ffn, const uint8_t* qu, const h16* su,
                                  const float* bup, const uint8_t* qg, const h16* sg, const float* bg,
                                  const uint8_t* qd, const h16* sd, const int32_t* idx, const int32_t* count,
                                  float* y, const FusedSparseLayout& L, char* hdr, char* data, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// q4.hip
hipError_t launch_quantize_rows(const h16* W, int rows, int d, uint8_t* q, h16* s, hipStream_t st);
hipError_t launch_ffn_q4(int kind, bool dense, const h16* x, int B, int d, int ffn, const uint8_t* qu,
                         const h16* su, const float* bup, const uint8_t* qg, const h16* sg, const float* bg,
                         const uint8_t* qd, const h16* sd, const int32_t* idx, const int32_t* count, float* y,
                         const SparseLayout& L, char* data, hipStream_t s);

// profile.hip
hipError_t launch_profile(const h16* X, int n, int d, int ffn, const h16* W, const float* b,
                          uint32_t* counts, hipStream_t s);
hipError_t launch_permute(const void* src, void* dst, int rows, int row_bytes,
                          const int32_t* perm, hipStream_t s);

}  // namespace pi
