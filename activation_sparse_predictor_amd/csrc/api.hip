// C ABI of the sparse-FFN library: argument validation, workspace layout and
// launches.  Every check runs before the first launch, so a rejected call
// leaves the device untouched.  See include/pi.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <numeric>
#include <unordered_map>
#include <vector>

#include "internal.hpp"
#include "pi.h"

namespace {

thread_local char g_err[512] = "";

pi_status fail(pi_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

pi_status ok() {
    g_err[0] = '\0';
    return PI_OK;
}

pi_status hip_fail(hipError_t e, const char* where) {
    return fail(PI_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

#define PI_REQUIRE(cond, status, ...) \
    do {                              \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

pi_status check_dims(int B, int d, int ffn) {
    PI_REQUIRE(B >= 1 && B <= PI_MAX_BATCH, PI_ERR_INVALID_ARG, "B=%d outside [1, %d]", B, PI_MAX_BATCH);
    PI_REQUIRE(d > 0 && ffn > 0, PI_ERR_INVALID_ARG, "d=%d ffn=%d must be positive", d, ffn);
    PI_REQUIRE(d % 8 == 0, PI_ERR_UNSUPPORTED, "d=%d is not a multiple of 8", d);
    PI_REQUIRE(d <= PI_MAX_D, PI_ERR_UNSUPPORTED, "d=%d above PI_MAX_D=%d", d, PI_MAX_D);
    PI_REQUIRE(ffn <= PI_MAX_FFN, PI_ERR_UNSUPPORTED, "ffn=%d above PI_MAX_FFN=%d", ffn, PI_MAX_FFN);
    return PI_OK;
}

pi_status check_half(const void* p, const char* name, bool required) {
    if (!p) return required ? fail(PI_ERR_INVALID_ARG, "%s is NULL", name) : PI_OK;
    PI_REQUIRE(aligned(p, 16), PI_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
    return PI_OK;
}

pi_status check_word(const void* p, const char* name, bool required) {
    if (!p) return required ? fail(PI_ERR_INVALID_ARG, "%s is NULL", name) : PI_OK;
    PI_REQUIRE(aligned(p, 4), PI_ERR_UNSUPPORTED, "%s is not 4-byte aligned", name);
    return PI_OK;
}

pi_status check_ws(void* ws, size_t ws_bytes, size_t need, const char* op) {
    if (need == 0) return PI_OK;
    PI_REQUIRE(ws != nullptr, PI_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", op, need);
    PI_REQUIRE(ws_bytes >= need, PI_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", op,
               ws_bytes, need);
    PI_REQUIRE(aligned(ws, 256), PI_ERR_UNSUPPORTED, "%s: workspace is not 256-byte aligned", op);
    return PI_OK;
}

// Every workspace starts with the fused kernels' synchronisation header; a
// call's data area follows it.
size_t predict_data_bytes(int B, int r, int ffn) {
    const size_t f = pi::fused_pred_layout(r, ffn).total;   // single token (and INT4 rows at any B)
    if (B == 1) return f;
    const size_t b = pi::bpred_layout(B < pi::kUnionMaxTokens ? B : pi::kUnionMaxTokens, r, ffn).total;
    return b > f ? b : f;
}
size_t predict_ws_bytes(int B, int r, int ffn) { return pi::kSyncBytes + predict_data_bytes(B, r, ffn); }

size_t sparse_data_bytes(int B, int d, int ffn) {
    size_t n = pi::sparse_layout(B, d, ffn).total;          // dense baseline
    const size_t f = pi::fused_sparse_layout(d, ffn).total;  // single token / per token
    if (f > n) n = f;
    if (B >= 2) {   // union path, by groups of kUnionMaxTokens and the last group (its chunk count may differ)
        const size_t u = pi::batch_layout(B < pi::kUnionMaxTokens ? B : pi::kUnionMaxTokens, d, ffn).total;
        if (u > n) n = u;
        const int tail = B % pi::kUnionMaxTokens;
        if (B > pi::kUnionMaxTokens && tail > 0) {
            const size_t ut = pi::batch_layout(tail, d, ffn).total;
            if (ut > n) n = ut;
        }
    }
    return n;
}
size_t sparse_ws_bytes(int B, int d, int ffn) { return pi::kSyncBytes + sparse_data_bytes(B, d, ffn); }

// pi_ffn_decode: one header, the predictor's data area, then the FFN's, so
// that repeated steps never find another layout in either area.
size_t decode_ffn_offset(int B, int r, int ffn) { return pi::kSyncBytes + pi::align256(predict_data_bytes(B, r, ffn)); }
size_t decode_ws_bytes(int B, int d, int r, int ffn) { return decode_ffn_offset(B, r, ffn) + sparse_data_bytes(B, d, ffn); }

// pi_ffn_decode_hot: the header, the predictor's data area, the hot prefix's
// area (its FFN inside the predictor's kernel), then the FFN's data area.
size_t decode_hot_area_offset(int B, int r, int ffn) { return decode_ffn_offset(B, r, ffn); }
size_t decode_hot_ffn_offset(int B, int d, int r, int ffn) {
    return decode_hot_area_offset(B, r, ffn) + pi::align256(pi::hot_layout(d, ffn).total);
}
size_t decode_hot_ws_bytes(int B, int d, int r, int ffn) {
    return decode_hot_ffn_offset(B, d, r, ffn) + sparse_data_bytes(B, d, ffn);
}

// Which layout each workspace last held, by its address.  Tags of earlier
// fused calls can never match a new epoch, but data written by another
// layout could, so a call that uses tagged words zeroes them whenever the
// workspace last held something else (another operation or shape, an
// unfused call, or a workspace not seen before).
struct LayoutKey {
    int op, B, d, r, ffn;
    bool operator==(const LayoutKey& o) const {
        return op == o.op && B == o.B && d == o.d && r == o.r && ffn == o.ffn;
    }
};
std::mutex g_ws_mu;
std::unordered_map<const void*, LayoutKey> g_ws_layout;

// true if the tagged words must be zeroed before a call with this layout
bool ws_needs_clear(const void* ws, const LayoutKey& key) {
    std::lock_guard<std::mutex> g(g_ws_mu);
    auto it = g_ws_layout.find(ws);
    return it == g_ws_layout.end() || !(it->second == key);
}
void ws_record(const void* ws, const LayoutKey& key) {
    std::lock_guard<std::mutex> g(g_ws_mu);
    g_ws_layout[ws] = key;
}
void ws_forget(const void* ws) {
    std::lock_guard<std::mutex> g(g_ws_mu);
    g_ws_layout.erase(ws);
}

// Whether a call's path keeps tagged words in its data area.
bool sparse_is_fused(int B, uint32_t flags) {
    return (flags & PI_DENSE) == 0u && (B == 1 || (flags & PI_PER_TOKEN) != 0u);
}

#define PI_TRY(expr)                  \
    do {                              \
        pi_status _s = (expr);        \
        if (_s != PI_OK) return _s;   \
    } while (0)

pi_status check_predict_args(const pi_half* x, int B, int d, const pi_half* P1, const float* b1, int act,
                             const pi_half* P2, const float* b2, int r, int ffn, float tau, const int32_t* idx,
                             const int32_t* count) {
    PI_TRY(check_dims(B, d, ffn));
    PI_REQUIRE(r > 0, PI_ERR_INVALID_ARG, "r=%d must be positive", r);
    PI_REQUIRE(r % 8 == 0, PI_ERR_UNSUPPORTED, "r=%d is not a multiple of 8", r);
    PI_REQUIRE(r <= PI_MAX_R, PI_ERR_UNSUPPORTED, "r=%d above PI_MAX_R=%d", r, PI_MAX_R);
    PI_REQUIRE(act == PI_ACT_RELU || act == PI_ACT_NONE, PI_ERR_INVALID_ARG, "act=%d unknown", act);
    PI_REQUIRE(tau > 0.f && tau < 1.f, PI_ERR_INVALID_ARG, "tau=%g not in (0, 1)", (double)tau);
    PI_TRY(check_half(x, "x", true));
    PI_TRY(check_half(P1, "P1", true));
    PI_TRY(check_half(P2, "P2", true));
    PI_TRY(check_word(b1, "b1", false));
    PI_TRY(check_word(b2, "b2", false));
    PI_TRY(check_word(idx, "idx", true));
    PI_TRY(check_word(count, "count", true));
    return PI_OK;
}

// The FFN's kind, weights and biases.
pi_status check_ffn_weights(int kind, const pi_half* W_up, const float* b_up, const pi_half* W_gate,
                            const float* b_gate, const pi_half* W_down) {
    PI_REQUIRE(kind == PI_FFN_RELU || kind == PI_FFN_REGLU || kind == PI_FFN_SWIGLU, PI_ERR_INVALID_ARG,
               "kind=%d unknown", kind);
    const bool gated = kind != PI_FFN_RELU;   // ReGLU and SwiGLU take a W_gate row per neuron
    PI_REQUIRE(gated == (W_gate != nullptr), PI_ERR_INVALID_ARG,
               gated ? "W_gate is NULL for a gated (ReGLU / SwiGLU) FFN" : "W_gate given for a ReLU FFN");
    PI_REQUIRE(gated || b_gate == nullptr, PI_ERR_INVALID_ARG, "b_gate given for a ReLU FFN");
    PI_TRY(check_half(W_up, "W_up", true));
    PI_TRY(check_half(W_gate, "W_gate", false));
    PI_TRY(check_half(W_down, "W_down", true));
    PI_TRY(check_word(b_up, "b_up", false));
    PI_TRY(check_word(b_gate, "b_gate", false));
    return PI_OK;
}

pi_status check_sparse_args(int kind, const pi_half* x, int B, int d, int ffn, const pi_half* W_up,
                            const float* b_up, const pi_half* W_gate, const float* b_gate, const pi_half* W_down,
                            const int32_t* idx, const int32_t* count, const float* y, uint32_t flags) {
    PI_TRY(check_dims(B, d, ffn));
    PI_REQUIRE(kind == PI_FFN_RELU || kind == PI_FFN_REGLU || kind == PI_FFN_SWIGLU, PI_ERR_INVALID_ARG,
               "kind=%d unknown", kind);
    PI_REQUIRE((flags & ~(PI_DENSE | PI_PER_TOKEN | PI_DETERMINISTIC | PI_CHECK_IDX)) == 0u, PI_ERR_INVALID_ARG,
               "unknown flags 0x%x", flags);
    const bool dense = (flags & PI_DENSE) != 0u;
    PI_TRY(check_ffn_weights(kind, W_up, b_up, W_gate, b_gate, W_down));
    PI_TRY(check_half(x, "x", true));
    PI_TRY(check_word(idx, "idx", !dense));
    PI_TRY(check_word(count, "count", !dense));
    PI_REQUIRE(y != nullptr, PI_ERR_INVALID_ARG, "y is NULL");
    PI_REQUIRE(aligned(y, 16), PI_ERR_UNSUPPORTED, "y is not 16-byte aligned");
    return PI_OK;
}


// The calls proper, on a checked workspace: hdr is its synchronisation header,
// data the call's data area; clear: zero the tagged words first (single-token
// paths only).
// sigmoid(z) > tau  <=>  z > ln(tau / (1 - tau)), evaluated once in double.
float logit_threshold(float tau) { return (float)std::log((double)tau / (1.0 - (double)tau)); }

pi_status run_predict(const pi_half* x, int B, int d, const pi_half* P1, const float* b1, int act,
                      const pi_half* P2, const float* b2, int r, int ffn, int hot, float tau, int32_t* idx,
                      int32_t* count, char* hdr, char* data, bool clear, hipStream_t s) {
    const float thr = logit_threshold(tau);
    const auto* hx = reinterpret_cast<const pi::h16*>(x);
    const auto* h1 = reinterpret_cast<const pi::h16*>(P1);
    const auto* h2 = reinterpret_cast<const pi::h16*>(P2);
    if (B >= 2) {   // batched: both predictor layers on the matrix cores, weights read once per group
        for (int g0 = 0; g0 < B; g0 += pi::kUnionMaxTokens) {
            const int Bg = B - g0 < pi::kUnionMaxTokens ? B - g0 : pi::kUnionMaxTokens;
            const pi::BPredLayout L = pi::bpred_layout(Bg, r, ffn);
            hipError_t e = pi::launch_bpredict(hx + (size_t)g0 * d, Bg, d, h1, b1, act == PI_ACT_RELU, h2, b2,
                                               r, ffn, hot, thr, idx + (size_t)g0 * ffn, count + g0, L,
                                               data, hdr, s);
            if (e != hipSuccess) return hip_fail(e, "pi_ffn_predict batched");
        }
        return ok();
    }
    // one token: a single kernel, hidden rows overlapping the logits tiles
    const pi::FusedPredLayout L = pi::fused_pred_layout(r, ffn);
    hipError_t e = hipSuccess;
    if (clear) e = pi::launch_zero(data, L.total, s);
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_predict clearing the workspace");
    e = pi::launch_predict_fused(hx, d, h1, b1, act == PI_ACT_RELU, r, h2, b2, ffn, hot, thr, L, hdr, data, idx,
                                 count, s);
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_predict");
    return ok();
}

pi_status run_sparse(int kind, const pi_half* x, int B, int d, int ffn, const pi_half* W_up, const float* b_up,
                     const pi_half* W_gate, const float* b_gate, const pi_half* W_down, const int32_t* idx,
                     const int32_t* count, float* y, uint32_t flags, char* hdr, char* data, bool clear,
                     hipStream_t s) {
    const bool dense = (flags & PI_DENSE) != 0u;
    const bool check = !dense && (flags & PI_CHECK_IDX) != 0u;
    const auto* hx = reinterpret_cast<const pi::h16*>(x);
    const auto* hu = reinterpret_cast<const pi::h16*>(W_up);
    const auto* hg = reinterpret_cast<const pi::h16*>(W_gate);
    const auto* hd = reinterpret_cast<const pi::h16*>(W_down);
    if (B >= 2 && !dense && !(flags & PI_PER_TOKEN)) {
        for (int g0 = 0; g0 < B; g0 += pi::kUnionMaxTokens) {
            const int Bg = B - g0 < pi::kUnionMaxTokens ? B - g0 : pi::kUnionMaxTokens;
            const pi::BatchLayout L = pi::batch_layout(Bg, d, ffn);
            hipError_t e = pi::launch_union(kind, hx + (size_t)g0 * d, Bg, d, ffn, hu, b_up, hg, b_gate, hd,
                                            idx + (size_t)g0 * ffn, count + g0, y + (size_t)g0 * d, L,
                                            data, hdr, s);
            if (e != hipSuccess) return hip_fail(e, "pi_ffn_sparse union path");
        }
        if (check) {
            hipError_t e = pi::launch_check_idx(idx, count, B, ffn, d, y, s);
            if (e != hipSuccess) return hip_fail(e, "pi_ffn_sparse index check");
        }
        return ok();
    }
    if (!dense) {   // one token (or PI_PER_TOKEN): one kernel per token, up/gate rows overlapping W_down
        const pi::FusedSparseLayout L = pi::fused_sparse_layout(d, ffn);
        hipError_t e = hipSuccess;
        if (clear) e = pi::launch_zero(data + L.atag, L.partial - L.atag, s);
        if (e != hipSuccess) return hip_fail(e, "pi_ffn_sparse clearing the workspace");
        for (int t = 0; t < B && e == hipSuccess; ++t)
            e = pi::launch_sparse_fused(kind, hx + (size_t)t * d, d, ffn, hu, b_up, hg, b_gate, hd,
                                        idx + (size_t)t * ffn, count + t, y + (size_t)t * d, L, hdr, data, s);
        if (e != hipSuccess) return hip_fail(e, "pi_ffn_sparse");
        if (check) {
            e = pi::launch_check_idx(idx, count, B, ffn, d, y, s);
            if (e != hipSuccess) return hip_fail(e, "pi_ffn_sparse index check");
        }
        return ok();
    }
    const pi::SparseLayout L = pi::sparse_layout(B, d, ffn);
    float* a = reinterpret_cast<float*>(data + L.a);
    float* partial = reinterpret_cast<float*>(data + L.partial);
    uint32_t* ctr = reinterpret_cast<uint32_t*>(data + L.ctr);
    hipError_t e = pi::launch_up_act(kind, dense, hx, B, d, ffn, hu, b_up, hg, b_gate, idx, count, a,
                                     ctr, L.T, s);
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_sparse up/gate");
    e = pi::launch_down_acc(dense, hd, B, d, ffn, idx, count, a, y, partial, ctr, L.T, L.G, s);
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_sparse down");
    return ok();
}

pi_status check_decode_args(int kind, const pi_half* x, int B, int d, int ffn, const pi_half* P1, const float* b1,
                            int act, const pi_half* P2, const float* b2, int r, float tau, const pi_half* W_up,
                            const float* b_up, const pi_half* W_gate, const float* b_gate, const pi_half* W_down,
                            const int32_t* idx, const int32_t* count, const float* y, uint32_t flags) {
    PI_TRY(check_predict_args(x, B, d, P1, b1, act, P2, b2, r, ffn, tau, idx, count));
    PI_TRY(check_sparse_args(kind, x, B, d, ffn, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags));
    PI_REQUIRE((flags & PI_DENSE) == 0u, PI_ERR_INVALID_ARG, "PI_DENSE has no predictor step: call pi_ffn_sparse");
    return PI_OK;
}

// One decode step on a checked workspace w of at least decode_ws_bytes() bytes.
pi_status decode_on(int kind, const pi_half* x, int B, int d, int ffn, const pi_half* P1, const float* b1, int act,
                    const pi_half* P2, const float* b2, int r, float tau, const pi_half* W_up, const float* b_up,
                    const pi_half* W_gate, const float* b_gate, const pi_half* W_down, int32_t* idx,
                    int32_t* count, float* y, uint32_t flags, char* w, hipStream_t s) {
    // one key for both data areas: where the FFN's starts depends on B, r and ffn
    const LayoutKey key{PI_OP_DECODE, B, d, r, ffn};
    const bool fused = B == 1 || sparse_is_fused(B, flags);
    const bool clear = fused && ws_needs_clear(w, key);
    if (!fused) ws_forget(w);
    PI_TRY(run_predict(x, B, d, P1, b1, act, P2, b2, r, ffn, 0, tau, idx, count, w, w + pi::kSyncBytes,
                       clear && B == 1, s));
    PI_TRY(run_sparse(kind, x, B, d, ffn, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags, w,
                      w + decode_ffn_offset(B, r, ffn), clear && sparse_is_fused(B, flags), s));
    if (fused) ws_record(w, key);
    return PI_OK;
}

// The two launches of a single-token hot decode step on a checked workspace w
// of at least decode_hot_ws_bytes(1, ...) bytes.  Begin: the predictor's kernel
// with the hot prefix's FFN in extra roles (its chunk partials left in the hot
// area); it clears the tagged words first when the workspace held another
// layout.  End: the FFN kernel over list positions [n_hot, count), adding the
// prefix's partials and advancing its epoch slots.
pi_status hot_begin_on(int kind, const pi_half* x, int d, int ffn, const pi_half* P1, const float* b1, int act,
                       const pi_half* P2, const float* b2, int r, int n_hot, float tau, const pi_half* W_up,
                       const float* b_up, const pi_half* W_gate, const float* b_gate, const pi_half* W_down,
                       int32_t* idx, int32_t* count, char* w, hipStream_t s) {
    const LayoutKey key{PI_OP_DECODE_HOT, 1, d, r, ffn};
    const bool clear = ws_needs_clear(w, key);
    const pi::FusedPredLayout PL = pi::fused_pred_layout(r, ffn);
    const pi::HotLayout HL = pi::hot_layout(d, ffn);
    const pi::FusedSparseLayout FL = pi::fused_sparse_layout(d, ffn);
    char* pdata = w + pi::kSyncBytes;
    char* hot = w + decode_hot_area_offset(1, r, ffn);
    char* fdata = w + decode_hot_ffn_offset(1, d, r, ffn);
    hipError_t e = hipSuccess;
    // the predictor's area, the hot area and the FFN's tagged words are contiguous
    if (clear) e = pi::launch_zero(pdata, (size_t)(fdata + FL.partial - pdata), s);
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_decode_hot clearing the workspace");
    e = pi::launch_predict_fused_hot(kind, reinterpret_cast<const pi::h16*>(x), d, reinterpret_cast<const pi::h16*>(P1),
                                     b1, act == PI_ACT_RELU, r, reinterpret_cast<const pi::h16*>(P2), b2, ffn, n_hot,
                                     logit_threshold(tau), PL, w, pdata, idx, count,
                                     reinterpret_cast<const pi::h16*>(W_up), b_up,
                                     reinterpret_cast<const pi::h16*>(W_gate), b_gate,
                                     reinterpret_cast<const pi::h16*>(W_down), HL, hot, s);
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_decode_hot predict");
    ws_record(w, key);
    return PI_OK;
}

pi_status hot_end_on(int kind, const pi_half* x, int d, int ffn, int r, int n_hot, const pi_half* W_up,
                     const float* b_up, const pi_half* W_gate, const float* b_gate, const pi_half* W_down,
                     const int32_t* idx, const int32_t* count, float* y, uint32_t flags, char* w, hipStream_t s) {
    const pi::FusedSparseLayout FL = pi::fused_sparse_layout(d, ffn);
    const pi::HotLayout HL = pi::hot_layout(d, ffn);
    char* fdata = w + decode_hot_ffn_offset(1, d, r, ffn);
    hipError_t e = pi::launch_sparse_fused(kind, reinterpret_cast<const pi::h16*>(x), d, ffn,
                                           reinterpret_cast<const pi::h16*>(W_up), b_up,
                                           reinterpret_cast<const pi::h16*>(W_gate), b_gate,
                                           reinterpret_cast<const pi::h16*>(W_down), idx, count, y, FL, w, fdata, s,
                                           n_hot, &HL, w + decode_hot_area_offset(1, r, ffn));
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_decode_hot sparse");
    if ((flags & PI_CHECK_IDX) != 0u) {
        e = pi::launch_check_idx(idx, count, 1, ffn, d, y, s);
        if (e != hipSuccess) return hip_fail(e, "pi_ffn_decode_hot index check");
    }
    return PI_OK;
}

// One decode step with an always-listed hot prefix on a checked workspace w
// of at least decode_hot_ws_bytes() bytes.  One token: begin then end.
// Several tokens: pi_ffn_predict_hot and pi_ffn_sparse as they are.
pi_status decode_hot_on(int kind, const pi_half* x, int B, int d, int ffn, const pi_half* P1, const float* b1,
                        int act, const pi_half* P2, const float* b2, int r, int n_hot, float tau,
                        const pi_half* W_up, const float* b_up, const pi_half* W_gate, const float* b_gate,
                        const pi_half* W_down, int32_t* idx, int32_t* count, float* y, uint32_t flags, char* w,
                        hipStream_t s) {
    if (B == 1) {
        PI_TRY(hot_begin_on(kind, x, d, ffn, P1, b1, act, P2, b2, r, n_hot, tau, W_up, b_up, W_gate, b_gate, W_down, idx,
                            count, w, s));
        PI_TRY(hot_end_on(kind, x, d, ffn, r, n_hot, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags, w, s));
        return ok();
    }
    const LayoutKey key{PI_OP_DECODE_HOT, B, d, r, ffn};
    const bool fused = sparse_is_fused(B, flags);
    const bool clear = fused && ws_needs_clear(w, key);
    if (!fused) ws_forget(w);
    PI_TRY(run_predict(x, B, d, P1, b1, act, P2, b2, r, ffn, n_hot, tau, idx, count, w, w + pi::kSyncBytes, false, s));
    PI_TRY(run_sparse(kind, x, B, d, ffn, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags, w,
                      w + decode_hot_ffn_offset(B, d, r, ffn), clear, s));
    if (fused) ws_record(w, key);
    return ok();
}

// ---- pi_ffn_decode_noalloc: the decode step's scratch in a static device array.
// Each GPU the library runs on holds its own copy (kStaticScratchBytes) until
// the process ends.  Host code never passes the array's name to a kernel: the
// name is a host-side stand-in, not the device address.  The address comes
// from hipGetSymbolAddress, once per device with that device current, and is
// kept per device.
constexpr size_t kStaticScratchBytes = PI_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

std::mutex g_scratch_mu;
char* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's scratch address.  The first call on a device looks it
// up and zero-fills the array on `s` with a fill kernel (the header's epochs
// and counters must start at zero; later calls keep what the last one left).
pi_status static_scratch(hipStream_t s, char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_decode_noalloc: hipGetDevice");
    PI_REQUIRE(dev >= 0 && dev < kMaxDevices, PI_ERR_UNSUPPORTED, "device %d outside [0, %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "pi_ffn_decode_noalloc: hipGetSymbolAddress(scratch)");
        e = pi::launch_zero(p, kStaticScratchBytes, s);
        if (e != hipSuccess) return hip_fail(e, "pi_ffn_decode_noalloc: zero-filling the scratch");
        g_scratch[dev] = static_cast<char*>(p);
    }
    *out = g_scratch[dev];
    return PI_OK;
}

}  // namespace

extern "C" {

const char* pi_status_string(pi_status s) {
    switch (s) {
        case PI_OK: return "PI_OK";
        case PI_ERR_INVALID_ARG: return "PI_ERR_INVALID_ARG";
        case PI_ERR_UNSUPPORTED: return "PI_ERR_UNSUPPORTED";
        case PI_ERR_WORKSPACE: return "PI_ERR_WORKSPACE";
        case PI_ERR_HIP: return "PI_ERR_HIP";
    }
    return "PI_ERR_UNKNOWN";
}

const char* pi_last_error(void) { return g_err; }

pi_status pi_workspace_size(int op, int B, int d, int r, int ffn, size_t* bytes) {
    PI_REQUIRE(bytes != nullptr, PI_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    switch (op) {
        case PI_OP_PREDICT:
            PI_TRY(check_dims(B, d, ffn));
            PI_REQUIRE(r > 0 && r <= PI_MAX_R, PI_ERR_INVALID_ARG, "r=%d outside [1, %d]", r, PI_MAX_R);
            *bytes = predict_ws_bytes(B, r, ffn);
            return ok();
        case PI_OP_SPARSE:
            PI_TRY(check_dims(B, d, ffn));
            *bytes = sparse_ws_bytes(B, d, ffn);
            return ok();
        case PI_OP_PROFILE:
            *bytes = 0;
            return ok();
        case PI_OP_DECODE:
            PI_TRY(check_dims(B, d, ffn));
            PI_REQUIRE(r > 0 && r <= PI_MAX_R, PI_ERR_INVALID_ARG, "r=%d outside [1, %d]", r, PI_MAX_R);
            *bytes = decode_ws_bytes(B, d, r, ffn);
            return ok();
        case PI_OP_DECODE_HOT:
            PI_TRY(check_dims(B, d, ffn));
            PI_REQUIRE(r > 0 && r <= PI_MAX_R, PI_ERR_INVALID_ARG, "r=%d outside [1, %d]", r, PI_MAX_R);
            *bytes = decode_hot_ws_bytes(B, d, r, ffn);
            return ok();
    }
    return fail(PI_ERR_INVALID_ARG, "unknown op %d", op);
}

pi_status pi_ffn_predict(const pi_half* x, int B, int d, const pi_half* P1, const float* b1,
                         int act, const pi_half* P2, const float* b2, int r, int ffn, float tau,
                         int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
    return pi_ffn_predict_hot(x, B, d, P1, b1, act, P2, b2, r, ffn, 0, tau, idx, count, ws, ws_bytes, stream);
}

pi_status pi_ffn_predict_hot(const pi_half* x, int B, int d, const pi_half* P1, const float* b1,
                             int act, const pi_half* P2, const float* b2, int r, int ffn, int n_hot, float tau,
                             int32_t* idx, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
    PI_TRY(check_predict_args(x, B, d, P1, b1, act, P2, b2, r, ffn, tau, idx, count));
    PI_REQUIRE(n_hot >= 0 && n_hot <= ffn, PI_ERR_INVALID_ARG, "n_hot=%d outside [0, ffn=%d]", n_hot, ffn);
    PI_REQUIRE(n_hot % 32 == 0, PI_ERR_UNSUPPORTED, "n_hot=%d is not a multiple of 32", n_hot);
    PI_TRY(check_ws(ws, ws_bytes, predict_ws_bytes(B, r, ffn), n_hot ? "pi_ffn_predict_hot" : "pi_ffn_predict"));
    char* w = static_cast<char*>(ws);
    const LayoutKey key{PI_OP_PREDICT, 1, 0, r, ffn};
    const bool fused = B == 1;
    const bool clear = fused && ws_needs_clear(ws, key);
    if (!fused) ws_forget(ws);
    PI_TRY(run_predict(x, B, d, P1, b1, act, P2, b2, r, ffn, n_hot, tau, idx, count, w, w + pi::kSyncBytes, clear,
                       static_cast<hipStream_t>(stream)));
    if (fused) ws_record(ws, key);
    return PI_OK;
}

pi_status pi_ffn_predict_q4(const pi_half* x, int B, int d, const uint8_t* q_P1, const pi_half* s_P1,
                            const float* b1, int act, const uint8_t* q_P2, const pi_half* s_P2, const float* b2,
                            int r, int ffn, int n_hot, float tau, int32_t* idx, int32_t* count, void* ws,
                            size_t ws_bytes, void* stream) {
    // the fp16 argument checks, with the code arrays standing in for the weight pointers
    PI_TRY(check_predict_args(x, B, d, reinterpret_cast<const pi_half*>(q_P1), b1, act,
                              reinterpret_cast<const pi_half*>(q_P2), b2, r, ffn, tau, idx, count));
    PI_REQUIRE(d % 64 == 0, PI_ERR_UNSUPPORTED, "d=%d is not a multiple of 64 (the INT4 group)", d);
    PI_REQUIRE(r % 64 == 0, PI_ERR_UNSUPPORTED, "r=%d is not a multiple of 64 (the INT4 group)", r);
    PI_REQUIRE(s_P1 != nullptr && s_P2 != nullptr, PI_ERR_INVALID_ARG, "a scale array is NULL");
    PI_REQUIRE(aligned(s_P1, 2) && aligned(s_P2, 2), PI_ERR_UNSUPPORTED, "a scale array is not 2-byte aligned");
    PI_REQUIRE(n_hot >= 0 && n_hot <= ffn, PI_ERR_INVALID_ARG, "n_hot=%d outside [0, ffn=%d]", n_hot, ffn);
    PI_REQUIRE(n_hot % 32 == 0, PI_ERR_UNSUPPORTED, "n_hot=%d is not a multiple of 32", n_hot);
    PI_TRY(check_ws(ws, ws_bytes, predict_ws_bytes(B, r, ffn), "pi_ffn_predict_q4"));
    char* hdr = static_cast<char*>(ws);
    char* data = hdr + pi::kSyncBytes;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // one single-token kernel per token, on the layout, header fields and
    // epochs of pi_ffn_predict's single-token path
    const LayoutKey key{PI_OP_PREDICT, 1, 0, r, ffn};
    const pi::FusedPredLayout L = pi::fused_pred_layout(r, ffn);
    const float thr = logit_threshold(tau);
    hipError_t e = hipSuccess;
    if (ws_needs_clear(ws, key)) e = pi::launch_zero(data, L.total, st);
    for (int t = 0; t < B && e == hipSuccess; ++t)
        e = pi::launch_predict_fused_q4(reinterpret_cast<const pi::h16*>(x) + (size_t)t * d, d, q_P1,
                                        reinterpret_cast<const pi::h16*>(s_P1), b1, act == PI_ACT_RELU, r, q_P2,
                                        reinterpret_cast<const pi::h16*>(s_P2), b2, ffn, n_hot, thr, L, hdr, data,
                                        idx + (size_t)t * ffn, count + t, st);
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_predict_q4");
    ws_record(ws, key);
    return ok();
}

pi_status pi_ffn_sparse(int kind, const pi_half* x, int B, int d, int ffn, const pi_half* W_up,
                        const float* b_up, const pi_half* W_gate, const float* b_gate,
                        const pi_half* W_down, const int32_t* idx, const int32_t* count, float* y,
                        uint32_t flags, void* ws, size_t ws_bytes, void* stream) {
    PI_TRY(check_sparse_args(kind, x, B, d, ffn, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags));
    PI_TRY(check_ws(ws, ws_bytes, sparse_ws_bytes(B, d, ffn), "pi_ffn_sparse"));
    char* w = static_cast<char*>(ws);
    const LayoutKey key{PI_OP_SPARSE, 1, d, 0, ffn};
    const bool fused = sparse_is_fused(B, flags);
    const bool clear = fused && ws_needs_clear(ws, key);
    if (!fused) ws_forget(ws);
    PI_TRY(run_sparse(kind, x, B, d, ffn, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags, w,
                      w + pi::kSyncBytes, clear, static_cast<hipStream_t>(stream)));
    if (fused) ws_record(ws, key);
    return PI_OK;
}

pi_status pi_ffn_decode(int kind, const pi_half* x, int B, int d, int ffn, const pi_half* P1, const float* b1,
                        int act, const pi_half* P2, const float* b2, int r, float tau, const pi_half* W_up,
                        const float* b_up, const pi_half* W_gate, const float* b_gate, const pi_half* W_down,
                        int32_t* idx, int32_t* count, float* y, uint32_t flags, void* ws, size_t ws_bytes,
                        void* stream) {
    PI_TRY(check_decode_args(kind, x, B, d, ffn, P1, b1, act, P2, b2, r, tau, W_up, b_up, W_gate, b_gate, W_down,
                             idx, count, y, flags));
    PI_TRY(check_ws(ws, ws_bytes, decode_ws_bytes(B, d, r, ffn), "pi_ffn_decode"));
    return decode_on(kind, x, B, d, ffn, P1, b1, act, P2, b2, r, tau, W_up, b_up, W_gate, b_gate, W_down, idx, count,
                     y, flags, static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

pi_status pi_ffn_decode_hot(int kind, const pi_half* x, int B, int d, int ffn, const pi_half* P1, const float* b1,
                            int act, const pi_half* P2, const float* b2, int r, int n_hot, float tau,
                            const pi_half* W_up, const float* b_up, const pi_half* W_gate, const float* b_gate,
                            const pi_half* W_down, int32_t* idx, int32_t* count, float* y, uint32_t flags, void* ws,
                            size_t ws_bytes, void* stream) {
    PI_TRY(check_decode_args(kind, x, B, d, ffn, P1, b1, act, P2, b2, r, tau, W_up, b_up, W_gate, b_gate, W_down,
                             idx, count, y, flags));
    PI_REQUIRE(n_hot >= 0 && n_hot <= ffn, PI_ERR_INVALID_ARG, "n_hot=%d outside [0, ffn=%d]", n_hot, ffn);
    PI_REQUIRE(n_hot % 32 == 0, PI_ERR_UNSUPPORTED, "n_hot=%d is not a multiple of 32", n_hot);
    PI_TRY(check_ws(ws, ws_bytes, decode_hot_ws_bytes(B, d, r, ffn), "pi_ffn_decode_hot"));
    return decode_hot_on(kind, x, B, d, ffn, P1, b1, act, P2, b2, r, n_hot, tau, W_up, b_up, W_gate, b_gate, W_down,
                         idx, count, y, flags, static_cast<char*>(ws), static_cast<hipStream_t>(stream));
}

pi_status pi_ffn_decode_hot_begin(int kind, const pi_half* x, int d, int ffn, const pi_half* P1, const float* b1,
                                  int act, const pi_half* P2, const float* b2, int r, int n_hot, float tau,
                                  const pi_half* W_up, const float* b_up, const pi_half* W_gate, const float* b_gate,
                                  const pi_half* W_down, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                                  void* stream) {
    PI_TRY(check_predict_args(x, 1, d, P1, b1, act, P2, b2, r, ffn, tau, idx, count));
    PI_TRY(check_ffn_weights(kind, W_up, b_up, W_gate, b_gate, W_down));
    PI_REQUIRE(n_hot >= 0 && n_hot <= ffn, PI_ERR_INVALID_ARG, "n_hot=%d outside [0, ffn=%d]", n_hot, ffn);
    PI_REQUIRE(n_hot % 32 == 0, PI_ERR_UNSUPPORTED, "n_hot=%d is not a multiple of 32", n_hot);
    PI_TRY(check_ws(ws, ws_bytes, decode_hot_ws_bytes(1, d, r, ffn), "pi_ffn_decode_hot_begin"));
    PI_TRY(hot_begin_on(kind, x, d, ffn, P1, b1, act, P2, b2, r, n_hot, tau, W_up, b_up, W_gate, b_gate, W_down, idx,
                        count, static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
    return ok();
}

pi_status pi_ffn_decode_hot_end(int kind, const pi_half* x, int d, int ffn, int r, int n_hot, const pi_half* W_up,
                                const float* b_up, const pi_half* W_gate, const float* b_gate, const pi_half* W_down,
                                const int32_t* idx, const int32_t* count, float* y, uint32_t flags, void* ws,
                                size_t ws_bytes, void* stream) {
    PI_TRY(check_sparse_args(kind, x, 1, d, ffn, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags));
    PI_REQUIRE((flags & (PI_DENSE | PI_PER_TOKEN)) == 0u, PI_ERR_INVALID_ARG,
               "pi_ffn_decode_hot_end takes PI_CHECK_IDX and PI_DETERMINISTIC only");
    PI_REQUIRE(r > 0 && r <= PI_MAX_R, PI_ERR_INVALID_ARG, "r=%d outside [1, %d]", r, PI_MAX_R);
    PI_REQUIRE(n_hot >= 0 && n_hot <= ffn, PI_ERR_INVALID_ARG, "n_hot=%d outside [0, ffn=%d]", n_hot, ffn);
    PI_REQUIRE(n_hot % 32 == 0, PI_ERR_UNSUPPORTED, "n_hot=%d is not a multiple of 32", n_hot);
    PI_TRY(check_ws(ws, ws_bytes, decode_hot_ws_bytes(1, d, r, ffn), "pi_ffn_decode_hot_end"));
    PI_TRY(hot_end_on(kind, x, d, ffn, r, n_hot, W_up, b_up, W_gate, b_gate, W_down, idx, count, y, flags,
                      static_cast<char*>(ws), static_cast<hipStream_t>(stream)));
    return ok();
}

pi_status pi_ffn_decode_noalloc(int kind, const pi_half* x, int B, int d, int ffn, const pi_half* P1,
                                const float* b1, int act, const pi_half* P2, const float* b2, int r, float tau,
                                const pi_half* W_up, const float* b_up, const pi_half* W_gate,
                                const float* b_gate, const pi_half* W_down, int32_t* idx, int32_t* count, float* y,
                                uint32_t flags, void* stream) {
    PI_TRY(check_decode_args(kind, x, B, d, ffn, P1, b1, act, P2, b2, r, tau, W_up, b_up, W_gate, b_gate, W_down,
                             idx, count, y, flags));
    const size_t need = decode_ws_bytes(B, d, r, ffn);
    PI_REQUIRE(need <= kStaticScratchBytes, PI_ERR_WORKSPACE,
               "pi_ffn_decode_noalloc: these sizes need %zu bytes of scratch, the static scratch holds %zu "
               "(call pi_ffn_decode with a workspace)", need, kStaticScratchBytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* w = nullptr;
    PI_TRY(static_scratch(s, &w));
    return decode_on(kind, x, B, d, ffn, P1, b1, act, P2, b2, r, tau, W_up, b_up, W_gate, b_gate, W_down, idx, count,
                     y, flags, w, s);
}

pi_status pi_quantize_rows(const pi_half* W, int rows, int d, uint8_t* q, pi_half* scales, void* stream) {
    PI_REQUIRE(rows >= 1 && rows <= PI_MAX_FFN, PI_ERR_INVALID_ARG, "rows=%d outside [1, %d]", rows, PI_MAX_FFN);
    PI_REQUIRE(d >= 1, PI_ERR_INVALID_ARG, "d=%d must be positive", d);
    PI_REQUIRE(d % 64 == 0, PI_ERR_UNSUPPORTED, "d=%d is not a multiple of 64 (the INT4 group)", d);
    PI_REQUIRE(d <= PI_MAX_D, PI_ERR_UNSUPPORTED, "d=%d above PI_MAX_D=%d", d, PI_MAX_D);
    PI_TRY(check_half(W, "W", true));
    PI_REQUIRE(q != nullptr && scales != nullptr, PI_ERR_INVALID_ARG, "q or scales is NULL");
    PI_REQUIRE(aligned(q, 16), PI_ERR_UNSUPPORTED, "q is not 16-byte aligned");
    PI_REQUIRE(aligned(scales, 2), PI_ERR_UNSUPPORTED, "scales is not 2-byte aligned");
    hipError_t e = pi::launch_quantize_rows(reinterpret_cast<const pi::h16*>(W), rows, d, q,
                                            reinterpret_cast<pi::h16*>(scales), static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pi_quantize_rows");
    return ok();
}

pi_status pi_ffn_sparse_q4(int kind, const pi_half* x, int B, int d, int ffn, const uint8_t* q_up,
                           const pi_half* s_up, const float* b_up, const uint8_t* q_gate, const pi_half* s_gate,
                           const float* b_gate, const uint8_t* q_down, const pi_half* s_down, const int32_t* idx,
                           const int32_t* count, float* y, uint32_t flags, void* ws, size_t ws_bytes,
                           void* stream) {
    // the fp16 argument checks, with the code arrays standing in for the weight pointers
    PI_TRY(check_sparse_args(kind, x, B, d, ffn, reinterpret_cast<const pi_half*>(q_up), b_up,
                             reinterpret_cast<const pi_half*>(q_gate), b_gate,
                             reinterpret_cast<const pi_half*>(q_down), idx, count, y, flags & ~PI_CHECK_IDX));
    PI_REQUIRE((flags & ~(PI_DENSE | PI_DETERMINISTIC)) == 0u, PI_ERR_INVALID_ARG,
               "flags 0x%x: only PI_DENSE and PI_DETERMINISTIC apply to INT4 rows", flags);
    PI_REQUIRE(d % 64 == 0, PI_ERR_UNSUPPORTED, "d=%d is not a multiple of 64 (the INT4 group)", d);
    PI_REQUIRE(s_up != nullptr && s_down != nullptr && (kind == PI_FFN_RELU || s_gate != nullptr),
               PI_ERR_INVALID_ARG, "a scale array is NULL");
    PI_REQUIRE(aligned(s_up, 2) && aligned(s_down, 2) && aligned(s_gate, 2), PI_ERR_UNSUPPORTED,
               "a scale array is not 2-byte aligned");
    PI_TRY(check_ws(ws, ws_bytes, sparse_ws_bytes(B, d, ffn), "pi_ffn_sparse_q4"));
    char* hdr = static_cast<char*>(ws);
    char* data = hdr + pi::kSyncBytes;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (B == 1 && (flags & PI_DENSE) == 0u) {
        // one token: the fused single-token kernel over INT4 rows (the layout,
        // header fields and epochs of pi_ffn_sparse's single-token path)
        const LayoutKey key{PI_OP_SPARSE, 1, d, 0, ffn};
        const pi::FusedSparseLayout LF = pi::fused_sparse_layout(d, ffn);
        hipError_t e = hipSuccess;
        if (ws_needs_clear(ws, key)) e = pi::launch_zero(data + LF.atag, LF.partial - LF.atag, st);
        if (e == hipSuccess)
            e = pi::launch_sparse_fused_q4(kind, reinterpret_cast<const pi::h16*>(x), d, ffn, q_up,
                                           reinterpret_cast<const pi::h16*>(s_up), b_up, q_gate,
                                           reinterpret_cast<const pi::h16*>(s_gate), b_gate, q_down,
                                           reinterpret_cast<const pi::h16*>(s_down), idx, count, y, LF, hdr, data, st);
        if (e != hipSuccess) return hip_fail(e, "pi_ffn_sparse_q4");
        ws_record(ws, key);
        return ok();
    }
    ws_forget(ws);
    const pi::SparseLayout L = pi::sparse_layout(B, d, ffn);
    hipError_t e = pi::launch_ffn_q4(kind, (flags & PI_DENSE) != 0u, reinterpret_cast<const pi::h16*>(x), B, d, ffn,
                                     q_up, reinterpret_cast<const pi::h16*>(s_up), b_up, q_gate,
                                     reinterpret_cast<const pi::h16*>(s_gate), b_gate, q_down,
                                     reinterpret_cast<const pi::h16*>(s_down), idx, count, y, L, data, st);
    if (e != hipSuccess) return hip_fail(e, "pi_ffn_sparse_q4");
    return ok();
}

pi_status pi_profile(const pi_half* X, int n, int d, int ffn, const pi_half* W_fire,
                     const float* b_fire, uint32_t* counts, void* ws, size_t ws_bytes,
                     void* stream) {
    (void)ws;
    (void)ws_bytes;
    PI_REQUIRE(n >= 1, PI_ERR_INVALID_ARG, "n=%d must be >= 1", n);
    PI_TRY(check_dims(1, d, ffn));
    PI_TRY(check_half(X, "X", true));
    PI_TRY(check_half(W_fire, "W_fire", true));
    PI_TRY(check_word(b_fire, "b_fire", false));
    PI_TRY(check_word(counts, "counts", true));
    hipError_t e = pi::launch_profile(reinterpret_cast<const pi::h16*>(X), n, d, ffn,
                                      reinterpret_cast<const pi::h16*>(W_fire), b_fire, counts,
                                      static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pi_profile");
    return ok();
}

pi_status pi_reorder(const uint32_t* counts, int ffn, double hot_share, int32_t* perm,
                     int32_t* hot_count) {
    PI_REQUIRE(counts && perm && hot_count, PI_ERR_INVALID_ARG, "NULL pointer argument");
    PI_REQUIRE(ffn > 0 && ffn <= PI_MAX_FFN, PI_ERR_INVALID_ARG, "ffn=%d outside [1, %d]", ffn, PI_MAX_FFN);
    PI_REQUIRE(hot_share > 0.0 && hot_share <= 1.0, PI_ERR_INVALID_ARG,
               "hot_share=%g not in (0, 1]", hot_share);
    std::vector<int32_t> order(ffn);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(),
                     [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
    uint64_t total = 0;
    for (int i = 0; i < ffn; ++i) total += counts[i];
    int32_t hot = 0;
    if (total > 0) {
        const double target = hot_share * (double)total;
        uint64_t running = 0;
        hot = ffn;
        for (int k = 0; k < ffn; ++k) {
            running += counts[order[k]];
            if ((double)running >= target) {
                hot = k + 1;
                break;
            }
        }
    }
    std::copy(order.begin(), order.end(), perm);
    *hot_count = hot;
    return ok();
}

pi_status pi_permute_rows(const void* src, void* dst, int rows, int row_bytes,
                          const int32_t* perm, void* stream) {
    PI_REQUIRE(src && dst && perm, PI_ERR_INVALID_ARG, "NULL pointer argument");
    PI_REQUIRE(rows > 0 && row_bytes > 0, PI_ERR_INVALID_ARG, "rows=%d row_bytes=%d must be positive",
               rows, row_bytes);
    PI_REQUIRE(row_bytes % 4 == 0, PI_ERR_UNSUPPORTED, "row_bytes=%d is not a multiple of 4", row_bytes);
    PI_REQUIRE(aligned(src, 4) && aligned(dst, 4) && aligned(perm, 4), PI_ERR_UNSUPPORTED,
               "pointers must be 4-byte aligned");
    const char* s0 = static_cast<const char*>(src);
    const char* d0 = static_cast<const char*>(dst);
    const size_t bytes = (size_t)rows * row_bytes;
    PI_REQUIRE(s0 + bytes <= d0 || d0 + bytes <= s0, PI_ERR_INVALID_ARG, "src and dst overlap");
    hipError_t e = pi::launch_permute(src, dst, rows, row_bytes, perm, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pi_permute_rows");
    return ok();
}

}  // extern "C"
