/*
 * pi.h -- C ABI of the MI355X (gfx950) neuron-aware sparse-FFN decode library.
 *
 * The operation follows the PowerInfer pages (egguo-blog reading report of
 * arXiv 2312.12456): an online predictor marks the FFN neurons expected to
 * fire for a token (Part A section 2.3, system module 3); a neuron-aware
 * operator computes only those neurons' rows, with no sparse format
 * (module 4, and section 4.3); an offline profiler counts how often each
 * neuron fires on general text (module 1, section 2.2) and the hot neurons,
 * the minority carrying 80% of activations, are placed first (section 2.3
 * "hot/cold neurons", section 3.1 finding 1).  On one GPU the hot/cold split
 * becomes a hot-first reorder of the rows.
 *
 * Conventions for every call:
 *  - pi_half is an IEEE binary16 bit pattern.  Matrices are row-major.  FFN
 *    weights are neuron-major: row i of W_up, W_gate and W_down belongs to
 *    neuron i and has length d.  All tensor arguments are DEVICE pointers
 *    unless marked "host".
 *  - The caller owns every buffer.  The library allocates nothing; scratch
 *    memory is a caller-provided device workspace of at least
 *    pi_workspace_size() bytes, 256-byte aligned, that must not be used by
 *    another call running concurrently.  Zero-fill a workspace once when it
 *    is allocated; after that it belongs to the library: pass it to any
 *    number of calls (of any operation and shape) and write nothing else into
 *    it, unless you zero-fill it again.  The library keeps synchronisation
 *    words in it between calls and remembers, by address, which layout each
 *    workspace last held (a call that finds a different one clears what it
 *    needs first, at the cost of one small extra kernel): a separate workspace
 *    per operation avoids those clears.  A call captured into a graph decides
 *    at capture whether it clears; so between the replays of a graph, a
 *    workspace the graph uses must not be passed to a call of another layout
 *    (another operation, shape or batch size).
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *    means the default stream).  Nothing is copied to the host: the active
 *    count stays in device memory and later kernels read it there.
 *  - Every argument check runs before any launch; on an error nothing is
 *    launched and pi_last_error() holds a thread-local description.
 *  - Results are deterministic: the same inputs give bitwise equal outputs.
 *  - Limits: 1 <= B <= PI_MAX_BATCH; d and r multiples of 8; d <= PI_MAX_D;
 *    r <= PI_MAX_R; 1 <= ffn <= PI_MAX_FFN; pi_half tensors 16-byte aligned;
 *    float / int tensors 4-byte aligned.
 */
#ifndef PI_H_
#define PI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t pi_half;

typedef enum pi_status {
    PI_OK = 0,
    PI_ERR_INVALID_ARG = 1,  /* NULL pointer, size or enum out of range, tau not in (0,1) */
    PI_ERR_UNSUPPORTED = 2,  /* d or r not a multiple of 8, misaligned pointer, size above a limit */
    PI_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than pi_workspace_size() */
    PI_ERR_HIP = 4           /* a HIP runtime call or launch failed; text in pi_last_error() */
} pi_status;

typedef enum pi_ffn_kind {
    PI_FFN_RELU = 0,   /* a_i = max(W_up[i].x + b_up_i, 0) */
    PI_FFN_REGLU = 1,  /* a_i = max(W_gate[i].x + b_gate_i, 0) * (W_up[i].x + b_up_i) */
    PI_FFN_SWIGLU = 2  /* a_i = SiLU(W_gate[i].x + b_gate_i) * (W_up[i].x + b_up_i),
                          SiLU(g) = g / (1 + exp(-g)): the SiLU-gated models of Part A
                          sections 2.3 and 4.4.  Their activations outside the list are
                          small rather than zero (sparsity there is the share of neurons
                          that can be dropped at a perplexity cost under 1%, about half),
                          so the sparse result approximates the dense one; which neurons
                          to list is the predictor's calibration */
} pi_ffn_kind;

typedef enum pi_pred_act {
    PI_ACT_RELU = 0,   /* predictor hidden layer h = max(P1 x + b1, 0) */
    PI_ACT_NONE = 1    /* h = P1 x + b1 (linear low-rank predictor) */
} pi_pred_act;

typedef enum pi_op {
    PI_OP_PREDICT = 0,
    PI_OP_SPARSE = 1,
    PI_OP_PROFILE = 2,
    PI_OP_DECODE = 3,
    PI_OP_DECODE_HOT = 4
} pi_op;

/* pi_ffn_sparse flags */
#define PI_DENSE 0x1u      /* ignore idx/count and compute every neuron (dense FFN baseline) */
#define PI_PER_TOKEN 0x2u  /* B >= 2: run every token through the single-token kernel instead of
                              the union path (same results up to rounding: the union path
                              rounds each activation to fp16 once) */
#define PI_DETERMINISTIC 0x4u  /* accepted for callers that ask for it: every path is deterministic
                                  already (fixed reduction orders, no floating-point atomics) */
#define PI_CHECK_IDX 0x8u  /* after the FFN, check each token's list against the contract
                              (count in [0, ffn], ids in [0, ffn), strictly ascending) on the
                              device and fill y_t with NaN when it breaks it; without the flag a
                              broken list gives unspecified y (ids are read clamped to [0, ffn),
                              so never an access outside the weights).  Ignored with PI_DENSE. */

#define PI_MAX_BATCH 256
#define PI_MAX_D 16384
#define PI_MAX_R 8192
#define PI_MAX_FFN (1 << 24)

/*
 * pi_ffn_predict -- which neurons fire for each token.
 *
 * Per token t (x_t = row t of x):
 *   h = act(P1 x_t + b1)            P1: r x d, b1: r floats or NULL (= 0)
 *   z = P2 h + b2                   P2: ffn x r, b2: ffn floats or NULL (= 0)
 *   neuron i is active  <=>  sigmoid(z_i) > tau  <=>  z_i > ln(tau / (1 - tau))
 * (the per-layer predictor MLP of Part A section 2.3, module 3).  h and z are
 * accumulated in fp32; h is never rounded to fp16.
 *
 * Outputs (device): idx[t * ffn + j], j < count[t], the active neurons of
 * token t in strictly ascending order; count[t] in [0, ffn].  Entries of idx
 * at j >= count[t] are left unspecified.  idx holds B * ffn int32, count B.
 * For B = 1 the call is one kernel (the hidden rows overlap the reads of
 * P2); if one of its bounded internal waits ever ran out, count is set to -1,
 * and pi_ffn_sparse (every path, pi_ffn_sparse_q4 too) answers a negative
 * count with y_t = NaN, so the failure cannot pass as a result.
 *
 * Errors: INVALID_ARG for NULL x/P1/P2/idx/count, B/d/r/ffn out of range,
 * act not a pi_pred_act, tau not in (0,1); UNSUPPORTED for d or r not a
 * multiple of 8, misalignment, sizes above the limits; WORKSPACE if ws is
 * NULL or ws_bytes < pi_workspace_size(PI_OP_PREDICT, B, d, r, ffn).
 */
pi_status pi_ffn_predict(const pi_half* x, int B, int d,
                         const pi_half* P1, const float* b1, int act,
                         const pi_half* P2, const float* b2, int r, int ffn,
                         float tau, int32_t* idx, int32_t* count,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * pi_ffn_predict_hot -- pi_ffn_predict on a hot-first layer whose first n_hot
 * neurons are always active.
 *
 * After the offline profile and the hot-first reorder (pi_profile,
 * pi_reorder, pi_permute_rows), the neurons at the front are the ones that
 * fire on nearly every token, the hot end of the power law that the
 * profiler and the placement of Part A section 2.3 (modules 1-2) single out
 * and preload.  Listing such neurons unconditionally is this library's use
 * of that split on one GPU: they bypass the predictor, so rows [0, n_hot) of
 * P2 and b2 are never read, and computing a neuron that turns out inactive
 * only adds its exact contribution.  The other neurons are predicted exactly
 * as pi_ffn_predict does:
 *   idx_t = [0, 1, ..., n_hot - 1] followed by the ascending i >= n_hot with z_i > ln(tau / (1 - tau)).
 * P2 and b2 still hold all ffn rows (the caller's layout does not change).
 * n_hot = 0 is pi_ffn_predict.  The workspace is pi_workspace_size(PI_OP_PREDICT, ...).
 *
 * Errors: as pi_ffn_predict, plus INVALID_ARG for n_hot outside [0, ffn],
 * and UNSUPPORTED for n_hot not a multiple of 32 (whole 32-neuron mask words).
 */
pi_status pi_ffn_predict_hot(const pi_half* x, int B, int d,
                             const pi_half* P1, const float* b1, int act,
                             const pi_half* P2, const float* b2, int r, int ffn, int n_hot,
                             float tau, int32_t* idx, int32_t* count,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * pi_ffn_sparse -- the neuron-aware FFN over the active rows only.
 *
 * Per token t, over j < count[t] with i = idx[t * ffn + j]:
 *   u_i = W_up[i].x_t + b_up_i ;  gated kinds: g_i = W_gate[i].x_t + b_gate_i
 *   a_i = max(u_i, 0) (RELU), max(g_i, 0) * u_i (REGLU), or SiLU(g_i) * u_i (SWIGLU)
 *   y_t = sum_j a_i * W_down[i, :]                (no output bias)
 * (the neuron-aware operator of Part A section 2.3 module 4 / section 4.3;
 * W_down is neuron-major so each active neuron is one contiguous row).
 * With flags & PI_DENSE, idx and count are ignored (may be NULL) and every
 * neuron is computed: the dense FFN.  Biases may be NULL (= 0).  W_gate must
 * be non-NULL for REGLU and SWIGLU and NULL for RELU.  Products are fp16 x fp16 with
 * fp32 accumulation; y is fp32, B x d, fully overwritten (count 0 gives 0;
 * a negative count[t], the predictor's overrun report, gives y_t = NaN).
 * idx must hold valid, strictly ascending neuron ids (as written by
 * pi_ffn_predict); the call does not re-check them unless flags has
 * PI_CHECK_IDX (then a token whose list breaks this gets y_t = NaN).
 *
 * For B = 1 (and for every token under PI_PER_TOKEN) the step is one kernel:
 * the up/gate rows of the list are computed while the W_down rows are already
 * being read, and each column block of y is summed over a fixed partition of
 * the list in a fixed order.
 *
 * For B >= 2 (unless PI_DENSE or PI_PER_TOKEN) the tokens are taken in
 * groups of up to 128: the union U of the group's lists is formed on the
 * device, the rows of U are read once, and the up/gate and W_down products
 * run on the matrix cores (fp16 x fp16 -> fp32; each activation a_i is
 * rounded once to fp16 for the W_down product, a relative error of at most
 * 2^-11 per term, about 2e-4 in y's relative L2 norm).  A neuron outside
 * token t's own list contributes exactly 0 to y_t, so y_t matches the
 * single-token result up to that rounding: the union changes which rows are
 * read, not what is computed (the batched decode of Part A section 4.4).  The union is formed
 * by one kernel with a bounded internal wait; were it ever to run out, every
 * token's y would be NaN.
 *
 * Errors: as pi_ffn_predict, plus INVALID_ARG for an unknown kind or flag,
 * or a W_gate that does not match the kind.
 */
pi_status pi_ffn_sparse(int kind, const pi_half* x, int B, int d, int ffn,
                        const pi_half* W_up, const float* b_up,
                        const pi_half* W_gate, const float* b_gate,
                        const pi_half* W_down,
                        const int32_t* idx, const int32_t* count,
                        float* y, uint32_t flags,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * pi_ffn_decode -- one decode step of the layer: pi_ffn_predict followed by
 * pi_ffn_sparse on its list (the predictor, then the neuron-aware operator on
 * the predicted neurons only: Part A section 2.3 modules 3 and 4).
 *
 * Arguments are those of the two calls, with the same meaning, layouts and
 * checks; idx and count are outputs (the predicted list, as pi_ffn_predict
 * writes it) and y is computed from them.  flags: as pi_ffn_sparse, except
 * PI_DENSE, which is INVALID_ARG here (a dense step has no predictor).
 *
 * The call is pi_ffn_predict then pi_ffn_sparse on the same stream, so its
 * results are bitwise theirs (two kernels for B = 1).  The workspace is split
 * between the two, each part laid out as that call's own workspace, so that
 * repeated steps never clear it.
 *
 * ws: at least pi_workspace_size(PI_OP_DECODE, B, d, r, ffn) bytes (the
 * workspace rules above apply).
 */
pi_status pi_ffn_decode(int kind, const pi_half* x, int B, int d, int ffn,
                        const pi_half* P1, const float* b1, int act,
                        const pi_half* P2, const float* b2, int r, float tau,
                        const pi_half* W_up, const float* b_up,
                        const pi_half* W_gate, const float* b_gate,
                        const pi_half* W_down,
                        int32_t* idx, int32_t* count, float* y, uint32_t flags,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * pi_ffn_decode_hot -- one decode step of a hot-first layer: pi_ffn_predict_hot
 * (neurons [0, n_hot) always listed, the rest predicted) followed by
 * pi_ffn_sparse on its list.
 *
 * After the offline profile and the hot-first reorder, the neurons at the
 * front fire on nearly every token: the hot neurons that the pages place
 * first and keep resident (Part A section 2.3, modules 1-2; Part B).  Their
 * rows do not depend on the prediction, so for a single token (B = 1) their
 * FFN runs inside the predictor's kernel, beside the predictor's weight
 * stream instead of behind it: extra workgroups compute a_i for i < n_hot
 * and accumulate sum_{i < n_hot} a_i W_down[i, :], and the FFN kernel that
 * follows takes the list from position n_hot on and adds that sum.
 *
 * Results: idx and count exactly as pi_ffn_predict_hot writes them (the
 * prefix, then the predicted neurons); y is the FFN over that whole list, as
 * pi_ffn_sparse computes it, up to the order of the fp32 sums (the prefix's
 * part is summed separately and added once per output).  For B >= 2 the call
 * is pi_ffn_predict_hot then pi_ffn_sparse (the union path), bitwise.
 * Arguments, flags and checks: as pi_ffn_decode, plus n_hot as in
 * pi_ffn_predict_hot (INVALID_ARG outside [0, ffn], UNSUPPORTED when not a
 * multiple of 32).  n_hot = 0 computes what pi_ffn_decode computes.
 *
 * ws: at least pi_workspace_size(PI_OP_DECODE_HOT, B, d, r, ffn) bytes (the
 * workspace rules above apply).
 */
pi_status pi_ffn_decode_hot(int kind, const pi_half* x, int B, int d, int ffn,
                            const pi_half* P1, const float* b1, int act,
                            const pi_half* P2, const float* b2, int r, int n_hot, float tau,
                            const pi_half* W_up, const float* b_up,
                            const pi_half* W_gate, const float* b_gate,
                            const pi_half* W_down,
                            int32_t* idx, int32_t* count, float* y, uint32_t flags,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * pi_ffn_decode_hot_begin / pi_ffn_decode_hot_end -- the two launches of
 * pi_ffn_decode_hot for one token (B = 1), as separate calls, so a caller can
 * put other work (or timing) between them.  begin: the prediction (idx,
 * count, as pi_ffn_predict_hot writes them) and the hot prefix's FFN, whose
 * chunk partials stay in ws; end: the FFN over list positions [n_hot, count)
 * plus the prefix's sum of those partials, into y.  end must follow its begin
 * (a second begin before end gives unspecified results) on the same
 * workspace with the same
 * layer, token, n_hot, idx and count, and no other call on that workspace in
 * between; begin followed by end computes exactly what pi_ffn_decode_hot
 * computes (bitwise).  flags of end: PI_CHECK_IDX, PI_DETERMINISTIC.
 * ws: pi_workspace_size(PI_OP_DECODE_HOT, 1, d, r, ffn) bytes for both.
 * Errors: as pi_ffn_decode_hot.
 */
pi_status pi_ffn_decode_hot_begin(int kind, const pi_half* x, int d, int ffn,
                                  const pi_half* P1, const float* b1, int act,
                                  const pi_half* P2, const float* b2, int r, int n_hot, float tau,
                                  const pi_half* W_up, const float* b_up,
                                  const pi_half* W_gate, const float* b_gate,
                                  const pi_half* W_down, int32_t* idx, int32_t* count,
                                  void* ws, size_t ws_bytes, void* stream);
pi_status pi_ffn_decode_hot_end(int kind, const pi_half* x, int d, int ffn, int r, int n_hot,
                                const pi_half* W_up, const float* b_up,
                                const pi_half* W_gate, const float* b_gate,
                                const pi_half* W_down, const int32_t* idx, const int32_t* count,
                                float* y, uint32_t flags, void* ws, size_t ws_bytes, void* stream);

/*
 * pi_ffn_decode_noalloc -- pi_ffn_decode for callers that cannot allocate
 * device memory (code being captured into a graph, tight serving loops,
 * harnesses that forbid allocation): the same step, arguments, checks and
 * results (bitwise), with no workspace argument.  Its scratch is a static
 * device array of PI_NOALLOC_SCRATCH_BYTES inside the library, one copy per
 * GPU, held until the process ends; the call allocates nothing.
 *
 * Limit: the sizes must need at most PI_NOALLOC_SCRATCH_BYTES of workspace
 * (pi_workspace_size(PI_OP_DECODE, B, d, r, ffn)); a single token (B = 1)
 * fits up to d = 16384 with ffn up to about 100 000 (d = 9216: about 270 000);
 * batched sizes mostly do not.  Larger sizes return PI_ERR_WORKSPACE before
 * anything is launched.
 *
 * Every call on one GPU shares that GPU's array and finds what the last call
 * left in it (the library clears what must start at zero, on the stream, the
 * first time a GPU is used and whenever the sizes change): calls that overlap
 * on one GPU (other streams, other host threads) race, so serialise them.
 */
#define PI_NOALLOC_SCRATCH_BYTES (4u << 20)
pi_status pi_ffn_decode_noalloc(int kind, const pi_half* x, int B, int d, int ffn,
                                const pi_half* P1, const float* b1, int act,
                                const pi_half* P2, const float* b2, int r, float tau,
                                const pi_half* W_up, const float* b_up,
                                const pi_half* W_gate, const float* b_gate,
                                const pi_half* W_down,
                                int32_t* idx, int32_t* count, float* y, uint32_t flags,
                                void* stream);

/*
 * pi_profile -- offline activation counts (Part A section 2.2 "offline
 * profiling data", section 2.3 module 1 and the neuron impact v_i = f_i).
 *
 *   counts[i] += #{ t < n : W_fire[i].X_t + b_fire_i > 0 }
 *
 * X: n x d calibration tokens; W_fire: ffn x d, the matrix whose output goes
 * through the ReLU (W_up for RELU FFNs, W_gate for REGLU); b_fire: ffn
 * floats or NULL.  counts (device, uint32, ffn) ACCUMULATES, so several
 * calls over chunks of calibration tokens sum up; zero it before the first.
 * Pre-activations are fp32 accumulations of fp16 products (matrix cores).
 * Errors: as above; n must be >= 1.  ws: pi_workspace_size(PI_OP_PROFILE, ...)
 * (currently 0 bytes; ws may be NULL).
 */
pi_status pi_profile(const pi_half* X, int n, int d, int ffn,
                     const pi_half* W_fire, const float* b_fire,
                     uint32_t* counts, void* ws, size_t ws_bytes, void* stream);

/*
 * pi_quantize_rows -- INT4 neuron rows (this library's own format).
 *
 * Part A section 3.1 of the pages reports the method with INT4 weights as
 * well as FP16; no format is given there, so this one is the library's.  Each row
 * of W (rows x d fp16, d % 64 == 0) is cut into groups of 64 weights.  Group
 * g gets one fp16 scale
 *   s = fp16(max |w| / 7)            (fp32 division, then round to nearest even)
 * and its weights become
 *   c = clamp(rint(w / s), -8, 7)    (fp32 division, rint rounds half to even; c = 0 when s = 0)
 * stored as the 4-bit code c + 8, two per byte: weight e of a row is the low
 * nibble of byte e / 2 for even e, the high nibble for odd e.  The weight the
 * FFN uses is (code - 8) * s.
 * Outputs (device, caller-owned): q, rows x d / 2 bytes (16-byte aligned);
 * scales, rows x d / 64 fp16.  Asynchronous on the stream; no workspace.
 * Errors: INVALID_ARG for rows or d out of range or a NULL pointer;
 * UNSUPPORTED for d not a multiple of 64, d > PI_MAX_D, or misalignment.
 */
pi_status pi_quantize_rows(const pi_half* W, int rows, int d, uint8_t* q, pi_half* scales, void* stream);

/*
 * pi_ffn_predict_q4 -- pi_ffn_predict_hot with the predictor's P1 and P2 as
 * INT4 rows (as written by pi_quantize_rows: q_P1 r x d / 2 code bytes with
 * s_P1 r x d / 64 fp16 scales, q_P2 ffn x r / 2 with s_P2 ffn x r / 64).
 *
 * Part A section 3.1 of the pages runs the method with INT4 weights; the
 * predictors of section 4.4 are part of the model's weights, so this
 * library quantises them like the FFN rows.  The computation is
 * pi_ffn_predict_hot's with every weight replaced by its dequantised value
 * (code - 8) * s:
 *   h = act(P1 x_t + b1),  z = P2 h + b2,  idx_t = [0, n_hot) then the
 *   ascending i >= n_hot with z_i > ln(tau / (1 - tau)).
 * h and z are fp32 accumulations; h is never rounded.  The two matrices take
 * (r d + ffn r) / 2 code bytes plus one fp16 per 64 weights, a quarter of
 * the fp16 predictor and a little more.
 * Each token is one kernel (the single-token design of pi_ffn_predict),
 * so B tokens are B launches on the stream; count[t] = -1 reports an
 * overrun of that kernel's bounded internal wait.  The workspace is
 * pi_workspace_size(PI_OP_PREDICT, B, d, r, ffn).
 *
 * Errors: as pi_ffn_predict_hot; UNSUPPORTED for d or r not a multiple of
 * 64; INVALID_ARG for a NULL scale array.
 */
pi_status pi_ffn_predict_q4(const pi_half* x, int B, int d,
                            const uint8_t* q_P1, const pi_half* s_P1, const float* b1, int act,
                            const uint8_t* q_P2, const pi_half* s_P2, const float* b2,
                            int r, int ffn, int n_hot, float tau,
                            int32_t* idx, int32_t* count,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * pi_ffn_sparse_q4 -- pi_ffn_sparse over INT4 rows of W_up, W_gate and W_down
 * (as written by pi_quantize_rows; q_* are the code arrays, s_* their scales).
 *
 * The same computation as pi_ffn_sparse with each weight replaced by its
 * dequantised value (code - 8) * s: per token, over the listed neurons,
 * a_i = act(u_i, g_i) and y = sum a_i W_down[i, :].  Products and sums are in
 * fp32.  An active neuron's three rows take 3 * (d / 2 + d / 32) bytes
 * instead of 3 * 2d.  Flags: PI_DENSE (every neuron), PI_DETERMINISTIC
 * (accepted; the path is deterministic).  The workspace is
 * pi_workspace_size(PI_OP_SPARSE, B, d, r, ffn), laid out as pi_ffn_sparse's.
 * One token with a list: one kernel, the single-token design of
 * pi_ffn_sparse over INT4 rows.  Otherwise two kernels, B tokens sharing
 * each launch (one grid row per token).
 * Errors: as pi_ffn_sparse; UNSUPPORTED for d not a multiple of 64; INVALID_ARG
 * for a NULL scale array of a matrix that is used, or another flag.
 */
pi_status pi_ffn_sparse_q4(int kind, const pi_half* x, int B, int d, int ffn,
                           const uint8_t* q_up, const pi_half* s_up, const float* b_up,
                           const uint8_t* q_gate, const pi_half* s_gate, const float* b_gate,
                           const uint8_t* q_down, const pi_half* s_down,
                           const int32_t* idx, const int32_t* count, float* y, uint32_t flags,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * pi_reorder -- HOST-ONLY hot-first order from profile counts.
 *
 * perm (host, ffn int32, new -> old) lists neurons by descending count, ties
 * in ascending original index.  *hot_count (host) is the smallest k such that
 * the first k sorted counts sum to at least hot_share * sum(counts), computed
 * in double precision; 0 when every count is 0.  hot_share in (0, 1]; the
 * pages' hot set is hot_share = 0.8 (Part A section 2.3).
 * Errors: INVALID_ARG for NULL pointers, ffn out of range, hot_share not in
 * (0, 1].  Deterministic; no HIP call.
 */
pi_status pi_reorder(const uint32_t* counts, int ffn, double hot_share,
                     int32_t* perm, int32_t* hot_count);

/*
 * pi_permute_rows -- dst[j, :] = src[perm[j], :] for j < rows (device).
 *
 * Applies a pi_reorder plan to any row-major tensor (W_up, W_gate, W_down,
 * P2: row_bytes = 2 * cols; biases: row_bytes = 4).  Out of place: src and
 * dst must not overlap.  perm is a device int32 array of length rows whose
 * entries lie in [0, rows).  row_bytes must be a multiple of 4 and both
 * pointers 16-byte aligned (4-byte when row_bytes is not a multiple of 16).
 * With perm[j] = j it is a plain copy.
 */
pi_status pi_permute_rows(const void* src, void* dst, int rows, int row_bytes,
                          const int32_t* perm, void* stream);

/* Workspace bytes that `op` needs for these sizes (op is a pi_op). */
pi_status pi_workspace_size(int op, int B, int d, int r, int ffn, size_t* bytes);

/* Static description of a status code. */
const char* pi_status_string(pi_status status);

/* Thread-local description of the last error returned on this thread. */
const char* pi_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PI_H_ */
