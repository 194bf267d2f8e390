// Internal launch interface and workspace layout of the sparse-FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pi {

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// ---- predictor: compaction tiles of 64 neurons (one wave-wide ballot each)
constexpr int kPredTile = 64;
inline int pred_tiles(int ffn) { return (ffn + kPredTile - 1) / kPredTile; }

struct PredictLayout {
    size_t h;        // B x r fp32 hidden activations
    size_t status;   // B x tiles uint32 look-back words, then B uint32 tickets
    size_t total;
    int tiles;
};

inline PredictLayout predict_layout(int B, int r, int ffn) {
    PredictLayout L;
    L.tiles = pred_tiles(ffn);
    L.h = 0;
    L.status = align256((size_t)B * r * 4);
    L.total = L.status + align256(((size_t)B * L.tiles + B) * 4);
    return L;
}

// ---- W_down accumulate: column tiles of 1024 (128 threads x 8 fp16) and
// G neuron chunks per tile, reduced in a fixed order (deterministic).
constexpr int kDownThreads = 128;
constexpr int kDownCols = kDownThreads * 8;
inline int down_tiles(int d) { return (d + kDownCols - 1) / kDownCols; }
inline int down_chunks(int d, int ffn) {
    int T = down_tiles(d);
    int G = 512 / T;
    if (G < 1) G = 1;
    if (G > ffn) G = ffn;
    return G;
}

struct SparseLayout {
    size_t a;        // B x ffn fp32 activations, in active-list order
    size_t partial;  // B x G x d fp32 per-chunk partial outputs
    size_t ctr;      // B x T uint32 arrival counters
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
    L.total = L.ctr + align256((size_t)B * L.T * 4);
    return L;
}

typedef _Float16 h16;

// predict.hip
hipError_t launch_pred_hidden(const h16* x, int B, int d, const h16* P1, const float* b1,
                              bool relu, int r, float* h, uint32_t* clear, int n_clear,
                              hipStream_t s);
hipError_t launch_pred_compact(const h16* P2, const float* b2, const float* h, int B, int r,
                               int ffn, float thr, uint32_t* status, uint32_t* tickets,
                               int32_t* idx, int32_t* count, hipStream_t s);

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
