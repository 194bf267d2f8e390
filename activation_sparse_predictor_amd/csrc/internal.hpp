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
inline int pred_tiles(int ffn) { return (ffn + kPredTile - 1) / kPredTile; }

struct PredictLayout {
    size_t h;        // B x r fp32 hidden activations
    size_t masks;    // B x tiles uint64 active-neuron bitmaps
    size_t ctr;      // B x kCtrWords uint32 arrival counters
    size_t total;
    int tiles;
};

inline PredictLayout predict_layout(int B, int r, int ffn) {
    PredictLayout L;
    L.tiles = pred_tiles(ffn);
    L.h = 0;
    L.masks = align256((size_t)B * r * 4);
    L.ctr = L.masks + align256((size_t)B * L.tiles * 8);
    L.total = L.ctr + align256((size_t)B * kCtrWords * 4);
    return L;
}

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

typedef _Float16 h16;

// predict.hip
hipError_t launch_pred_hidden(const h16* x, int B, int d, const h16* P1, const float* b1,
                              bool relu, int r, float* h, uint32_t* ctr, hipStream_t s);
hipError_t launch_pred_compact(const h16* P2, const float* b2, const float* h, int B, int r,
                               int ffn, float thr, uint64_t* masks, uint32_t* ctr, int32_t* idx, int32_t* count, hipStream_t s);

// sparse.hip
hipError_t launch_up_act(bool reglu, bool dense, const h16* x, int B, int d, int ffn,
                         const h16* Wup, const float* bup, const h16* Wg, const float* bg,
                         const int32_t* idx, const int32_t* count, float* a, uint32_t* ctr,
                         int T, hipStream_t s);
hipError_t launch_down_acc(bool dense, const h16* Wd, int B, int d, int ffn, const int32_t* idx,
                           const int32_t* count, const float* a, float* y, float* partial,
                           uint32_t* ctr, int T, int G, hipStream_t s);

// profile.hip
hipError_t launch_profile(const h16* X, int n, int d, int ffn, const h16* W, const float* b,
                          uint32_t* counts, hipStream_t s);
hipError_t launch_permute(const void* src, void* dst, int rows, int row_bytes,
                          const int32_t* perm, hipStream_t s);

}  // namespace pi
