/*
 * moe.h -- C ABI of one GPU's MoE-layer forward on MI355X (gfx950).
 *
 * The layer: a router GEMM and static top-k softmax gating pick k of E
 * experts per token; compact per-expert dispatch queues are built by a
 * counting sort (histogram, exclusive scan, stable scatter), so that no
 * dense token-by-expert matrix is ever formed; each expert runs a bias-free
 * SwiGLU feed-forward over its queue; a gate-weighted combine returns the
 * results to token order.
 *
 * Sources (summaries of three papers; they give the structure, not the
 * formulas):
 *   - MoEBlaze summary (euno.news, "MoEBlaze: breaking the memory wall for
 *     efficient MoE training on modern GPUs"), Methodology item 1
 *     (data-structure-based dispatch through per-expert queues built during
 *     the forward pass and dropped after it), Methodology item 2 (dispatch
 *     and reverse dispatch fused around the expert FFN), Limitations (static
 *     top-k routing).
 *   - Piper technical summary (gist.science, Dutch), section 1 (problem
 *     statement): tall-and-skinny expert GEMMs and skewed expert loads.
 *   - DisagMoE technical summary (gist.science, Korean), section 2.2
 *     (AF-Pipe): k, the number of experts per token.
 *
 * Conventions shared by every entry point
 *   - Sizes: T tokens, hidden size d, E experts, k experts per token, SwiGLU
 *     width f.  An assignment is a = t*k + j (token t, slot j < k).
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; arrays
 *     are dense and row-major.  Weights use the [out, in] layout, so every
 *     GEMM operand is contiguous along its reduction dimension:
 *       x [T, d], w_router [E, d], w_gate [E, f, d], w_up [E, f, d],
 *       w_down [E, d, f], y [T, d], x_perm / y_perm [T*k, d].
 *     x, weights, x_perm, y_perm and y have the problem's dtype; logits and
 *     gates are float32; ids, counts, offsets and permutations are int32.
 *   - Device pointers must be 16-byte aligned.
 *   - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *     enqueued on it; no entry point synchronises, allocates or frees, and
 *     apart from moe_dispatch_no_alloc's static scratch the library keeps no
 *     mutable global state, so calls on different streams with different
 *     buffers may run concurrently.
 *   - Workspace `ws` (device, >= the size from moe_workspace_size) is
 *     scratch whose contents are undefined before and after the call; it
 *     must not be shared by calls that may overlap.
 *   - Status is returned synchronously.  All argument checks happen before
 *     any HIP call: MOE_ERR_INVALID_ARGUMENT (NULL required pointer, T < 0,
 *     d/E/k/f < 1, k > E, unknown dtype), MOE_ERR_UNSUPPORTED (outside the
 *     documented limits below, or a misaligned pointer),
 *     MOE_ERR_WORKSPACE_TOO_SMALL.  T == 0 is a valid no-op.  A failed
 *     kernel launch returns MOE_ERR_HIP; faults during execution surface on
 *     the stream.  Logits must be finite (not checked).
 *   - Limits: 1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E, MOE_MAX_TOPK),
 *     T*k <= 2^31 - 1 and T <= 2^24 - 1 (a kernel launch counts its
 *     work-items in 32 bits, and the per-token kernels run 256 lanes per
 *     token); bf16 needs d and f to be multiples of 64 and d*f <= 2^31 - 1
 *     (one expert's weight matrix below 4 GiB).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 32

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4
} moe_status_t;

typedef enum {
    MOE_DTYPE_F32 = 0,  /* float32 storage and arithmetic throughout */
    MOE_DTYPE_BF16 = 1  /* bf16 storage, bf16 MFMA products, fp32 accumulate */
} moe_dtype_t;

/* Which call a workspace size is asked for. */
typedef enum {
    MOE_OP_DISPATCH = 1,
    MOE_OP_EXPERT_FFN = 2,
    MOE_OP_FORWARD = 3,
    MOE_OP_BACKWARD = 4,
    MOE_OP_EXPERT_FFN_FP8 = 5
} moe_op_t;

/* The problem statement: T tokens, hidden size d, E experts, top-k, SwiGLU
 * width f, storage dtype (a moe_dtype_t value). */
typedef struct {
    int64_t T;
    int32_t d;
    int32_t E;
    int32_t k;
    int32_t f;
    int32_t dtype;
} moe_problem_t;

/* Optional outputs of moe_forward.  Any field may be NULL; a NULL field is
 * kept in the workspace instead.  Shapes as in moe_route / moe_dispatch. */
typedef struct {
    float* logits;           /* [T, E] router logits (not written when logits_in is given) */
    int32_t* topk_ids;       /* [T, k] */
    float* topk_gates;       /* [T, k] */
    int32_t* counts;         /* [E] */
    int32_t* offsets;        /* [E + 1] */
    int32_t* sorted_assign;  /* [T*k] */
    int32_t* assign_pos;     /* [T*k] */
    void* y_perm;            /* [T*k, d] expert outputs (moe_backward does not need them) */
} moe_forward_outputs_t;

/* The forward state moe_backward reads (from moe_forward's outputs). */
typedef struct {
    const int32_t* topk_ids;      /* [T, k] */
    const float* topk_gates;      /* [T, k] */
    const int32_t* offsets;       /* [E + 1] */
    const int32_t* sorted_assign; /* [T*k] */
    const int32_t* assign_pos;    /* [T*k] */
    const void* y_perm;           /* [T*k, d]; not read (may be NULL) */
} moe_forward_state_t;

/* Gradients moe_backward writes.  dx, dw_gate, dw_up and dw_down are
 * required; dw_router is required exactly when w_router is given; dlogits
 * is optional.  Weight gradients in the problem dtype, dlogits fp32. */
typedef struct {
    void* dx;          /* [T, d] */
    void* dw_gate;     /* [E, f, d] */
    void* dw_up;       /* [E, f, d] */
    void* dw_down;     /* [E, d, f] */
    void* dw_router;   /* [E, d] */
    float* dlogits;    /* [T, E] */
} moe_backward_outputs_t;

/* Expert weights quantised for moe_expert_ffn_fp8 (moe_quantize_weights_fp8
 * writes them; caller-owned device buffers): OCP FP8 E4M3 codes, one byte
 * per element, in the layouts of the bf16 weights, and one power-of-two
 * scale exponent per weight row (value ~= 2^exp[row] * code value). */
typedef struct {
    void* w_gate;          /* [E, f, d] codes */
    int32_t* w_gate_exp;   /* [E, f] */
    void* w_up;            /* [E, f, d] codes */
    int32_t* w_up_exp;     /* [E, f] */
    void* w_down;          /* [E, d, f] codes */
    int32_t* w_down_exp;   /* [E, d] */
} moe_fp8_weights_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(int32_t status);

/* Library ABI version (bumped when a signature changes). */
int32_t moe_abi_version(void);

/* Bytes of device workspace `op` needs for problem `p` (0 is possible).
 * Host only; no HIP call. */
moe_status_t moe_workspace_size(const moe_problem_t* p, int32_t op, size_t* bytes);

/*
 * moe_route -- router GEMM and static top-k gating.
 * The router picks a few experts for every token (Piper, Japanese
 * explainer, opening section); the policy is static top-k (MoEBlaze
 * summary, Limitations).
 *   logits[t, e] = sum_c x[t, c] * w_router[e, c]   (fp32 accumulate)
 *   topk_ids[t, j]: the k largest logits of token t in descending order,
 *     equal logits broken toward the lower expert id (-0.0 == +0.0).
 *   topk_gates[t, j] = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the k
 *     chosen logits (softmax renormalised over the chosen experts), fp32.
 * If logits_in [T, E] is non-NULL the router GEMM is skipped and x,
 * w_router and logits_out may be NULL (logits_out is ignored).  Otherwise x,
 * w_router and logits_out [T, E] are required and logits_out receives the
 * router logits that the selection then reads.  The selection is exact on
 * the fp32 logits, so ids are reproducible bit for bit from the same logits.
 */
moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_router,
                       const float* logits_in, float* logits_out,
                       int32_t* topk_ids, float* topk_gates, void* stream);

/*
 * moe_dispatch -- the dispatch queues (MoEBlaze summary, Methodology 1): a
 * stable counting sort of the assignments a = t*k + j by expert id.
 *   counts[e] = #{a : topk_ids[a] == e}
 *   offsets[0] = 0, offsets[e + 1] = offsets[e] + counts[e]
 *   sorted_assign[pos] = a, assign_pos[a] = pos, where the queue of expert e
 *     is positions [offsets[e], offsets[e+1]) in ascending a (stable).
 *   x_perm[pos, :] = x[sorted_assign[pos] / k, :] (bitwise row copy), only
 *     when x_perm is non-NULL (x is then required).
 * Workspace: moe_workspace_size(p, MOE_OP_DISPATCH).  All outputs are
 * bit-exact functions of topk_ids.
 */
moe_status_t moe_dispatch(const moe_problem_t* p, const int32_t* topk_ids, const void* x,
                          int32_t* counts, int32_t* offsets,
                          int32_t* sorted_assign, int32_t* assign_pos, void* x_perm,
                          void* ws, size_t ws_bytes, void* stream);

/* Bytes of the static device scratch moe_dispatch_no_alloc uses on each GPU. */
#define MOE_NO_ALLOC_SCRATCH_BYTES (1u << 20)

/*
 * moe_dispatch_no_alloc -- moe_dispatch for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments as
 * moe_dispatch without ws / ws_bytes, and the same outputs, bit for bit.
 * Its scratch (the per-block expert count table, whose size
 * moe_workspace_size(p, MOE_OP_DISPATCH) gives) lives in a static device
 * array of MOE_NO_ALLOC_SCRATCH_BYTES that each GPU holds until the process
 * ends; the call allocates and frees nothing.  A problem whose table does
 * not fit returns MOE_ERR_UNSUPPORTED before any HIP call (with 256
 * experts, up to about 8.4 M assignments T*k fit; with 128, twice that).
 * The first call on a GPU looks up the array's address there (once per
 * device, briefly making that device current); a failed lookup returns
 * MOE_ERR_HIP.  Every call on one GPU uses that GPU's one array, which keeps
 * the last call's contents (each call writes all it reads): calls that may
 * overlap on one GPU, on different streams or from unsynchronised threads,
 * race and must not be issued.
 */
moe_status_t moe_dispatch_no_alloc(const moe_problem_t* p, const int32_t* topk_ids, const void* x,
                                   int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                                   int32_t* assign_pos, void* x_perm, void* stream);

/*
 * moe_expert_ffn -- grouped SwiGLU expert FFN over the queues (the
 * tall-and-skinny expert GEMMs of the Piper summary, section 1):
 *   for every expert e and queue row pos in [offsets[e], offsets[e+1]):
 *     row = x_perm[pos] if x_perm != NULL, else x[sorted_assign[pos] / k]
 *     h = silu(w_gate[e] row) * (w_up[e] row),  silu(u) = u / (1 + e^-u)
 *     y_perm[pos] = w_down[e] h
 * With x_perm == NULL the row gather is fused into the first GEMM's operand
 * loads (MoEBlaze summary, Methodology 2); then x and sorted_assign are
 * required.  bf16: products on bf16 MFMA with fp32 accumulation, h rounded
 * to bf16 between the two GEMMs, y_perm rounded to bf16.  f32: fp32 FMA.
 * Workspace: moe_workspace_size(p, MOE_OP_EXPERT_FFN) (holds h).
 */
moe_status_t moe_expert_ffn(const moe_problem_t* p, const void* x_perm, const void* x,
                            const int32_t* sorted_assign, const int32_t* offsets,
                            const void* w_gate, const void* w_up, const void* w_down,
                            void* y_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine -- gate-weighted reverse dispatch (MoEBlaze summary,
 * Methodology 2):
 *   y[t, :] = sum_j topk_gates[t, j] * y_perm[assign_pos[t*k + j], :]
 * fp32 accumulation in ascending j, one rounding to the dtype per element;
 * every y row is written exactly once (deterministic).
 */
moe_status_t moe_combine(const moe_problem_t* p, const void* y_perm, const int32_t* assign_pos,
                         const float* topk_gates, void* y, void* stream);

/*
 * moe_forward -- the whole layer on one stream with no host
 * synchronisation: moe_route, moe_dispatch (queues only), moe_expert_ffn
 * with the gather fused, moe_combine.  logits_in (optional, [T, E]) skips
 * the router GEMM; otherwise x and w_router are used.  `out` (optional)
 * exposes intermediates.  Workspace: moe_workspace_size(p, MOE_OP_FORWARD).
 */
moe_status_t moe_forward(const moe_problem_t* p, const void* x, const void* w_router,
                         const float* logits_in, const void* w_gate, const void* w_up,
                         const void* w_down, void* y, const moe_forward_outputs_t* out,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * moe_backward_weights -- the weight layouts moe_backward's GEMMs read:
 *   w_down_t [E, f, d] = W_down transposed per expert,
 *   w_gu_t   [E, d, 2f]: row c holds W_gate[e][:, c] then W_up[e][:, c].
 * The weights change only at an optimizer step, so a caller computes these
 * once per step and keeps them (caller-owned device buffers).  bf16 only
 * (MOE_ERR_UNSUPPORTED otherwise); T is not used.
 */
moe_status_t moe_backward_weights(const moe_problem_t* p, const void* w_gate, const void* w_up,
                                  const void* w_down, void* w_down_t, void* w_gu_t, void* stream);

/*
 * moe_backward -- gradients of the layer for the output gradient dy [T, d]
 * (MoEBlaze summary, Methodology item 2: the backward runs on the
 * forward's dispatch queues; its checkpoint bullet and Key contributions
 * bullet 3: intermediates are recomputed rather than stored, here the SwiGLU
 * ones, from x).  Given the forward state `fw` (ids, gates, queues; its
 * y_perm is not read: the slot gradients come from the recompute) it
 * computes, with the routing held fixed:
 *   slot gradients dg = <dy[t], y_perm[pos]> (computed as <dy[t] W_down,
 *   h> from the recomputed h), per expert and queue row q
 *   (token t, gate g) dh = g dy[t] W_down, the recomputed u = x[t] W_gate^T,
 *   v = x[t] W_up^T with du = dh v silu'(u) and dv = dh silu(u), dx_perm =
 *   du W_gate + dv W_up, dx[t] = sum_j dx_perm[pos(t, j)] (+ the router
 *   term), dW_down = sum_q (g dy[t])^T h, dW_gate = sum_q du^T x[t],
 *   dW_up = sum_q dv^T x[t] (x and dy are read by token: no copy of either
 *   is made in queue order), the logit gradient of the renormalised top-k
 *   softmax
 *   dl_j = g_j (dg_j - sum_i g_i dg_i) (zero for experts outside the top k),
 *   and, with a router, dW_r = dl^T x and dx += dl W_r.
 * w_down_t and w_gu_t come from moe_backward_weights.  w_router is NULL
 * when the forward took supplied logits (then no router gradients).
 * bf16 only; needs d*f < 2^30, T*d < 2^31 and Kpad <= 2^31 - 1
 * (Kpad = T*k + 63*E rounded up to 64: the queues with each expert's start
 * padded to a multiple of 64, the blocks of the router gradient's partial
 * sums); MOE_ERR_UNSUPPORTED otherwise.  With T = 0 neither x, dy, dx nor the
 * fields of fw are read and the weight gradients come out zero.  Workspace:
 * moe_workspace_size(p, MOE_OP_BACKWARD).  Deterministic: every reduction
 * runs in a fixed order.
 */
moe_status_t moe_backward(const moe_problem_t* p, const void* x, const void* w_router,
                          const void* w_gate, const void* w_up, const void* w_down_t,
                          const void* w_gu_t, const moe_forward_state_t* fw, const void* dy,
                          const moe_backward_outputs_t* out, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * moe_quantize_rows_fp8 -- per-row FP8 quantisation of a bf16 matrix
 * src [rows, cols] (quantised experts: MoEBlaze summary, Limitations and
 * future work; the scheme is this library's reading).  Row r gets the
 * power-of-two scale 2^exps[r], the smallest with max|row| <= 448 * 2^exps[r]
 * (0 for an all-zero row), and codes[r, c] = E4M3(src[r, c] / 2^exps[r]),
 * OCP FP8 E4M3, rounded to nearest even.  cols must be a positive multiple
 * of 16 and rows at most 2^24 - 1 (MOE_ERR_UNSUPPORTED otherwise); src,
 * codes and exps 16-byte aligned.  rows = 0 is a no-op.
 */
moe_status_t moe_quantize_rows_fp8(const void* src, int64_t rows, int32_t cols, void* codes, int32_t* exps,
                                   void* stream);

/*
 * moe_quantize_weights_fp8 -- moe_quantize_rows_fp8 over every weight row
 * of W_gate, W_up [E, f, d] and W_down [E, d, f] into `out`.  Once per
 * weight update.  Needs bf16 with d and f multiples of 128.
 */
moe_status_t moe_quantize_weights_fp8(const moe_problem_t* p, const void* w_gate, const void* w_up,
                                      const void* w_down, const moe_fp8_weights_t* out, void* stream);

/*
 * moe_expert_ffn_fp8 -- moe_expert_ffn with fp8 GEMMs: x [T, d] bf16 is
 * quantised per token, GEMM1 multiplies its codes (gathered through
 * sorted_assign) with the codes of W_gate and W_up on FP8 MFMA with fp32
 * accumulation, applies both scales exactly and the SwiGLU, rounds h to
 * bf16 and quantises it in its epilogue, one power-of-two scale per block of
 * 32 columns of a queue row (an E8M0 byte, so at least 2^-127); GEMM2
 * multiplies the h codes with the codes of W_down on the block-scaled FP8
 * MFMA, which applies the h scales, then the W_down row scales, writing
 * y_perm [T*k, d] bf16.  Weights from moe_quantize_weights_fp8.
 * bf16 problems with d and f multiples of 128 and T*d < 2^32 only.
 * Workspace: moe_workspace_size(p, MOE_OP_EXPERT_FFN_FP8).
 */
moe_status_t moe_expert_ffn_fp8(const moe_problem_t* p, const void* x, const int32_t* sorted_assign,
                                const int32_t* offsets, const moe_fp8_weights_t* w, void* y_perm, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * moe_mfma_peak -- measurement kernel, not part of the layer: `workgroups`
 * workgroups of 4 waves each run `iters` rounds of 8 independent bf16
 * 32x32x16 MFMAs on register operands (no memory traffic), i.e.
 * workgroups * 4 * iters * 8 * 32768 FLOP, and write one float per
 * workgroup to sink [workgroups].  Timed by the caller, it gives the MFMA
 * rate this GPU sustains (its clock under full matrix load), the ceiling
 * the expert GEMMs are also reported against.  workgroups and iters must be
 * positive.
 */
moe_status_t moe_mfma_peak(int32_t workgroups, int32_t iters, float* sink, void* stream);

/*
 * moe_stream_copy -- measurement kernel, not part of the layer: dst[i] =
 * src[i] for `bytes` bytes, read and written once in 16-byte words
 * (non-overlapping device buffers, 16-byte aligned, bytes a multiple of 16:
 * MOE_ERR_UNSUPPORTED otherwise; bytes = 0 is a no-op).  Timed by the
 * caller, 2 * bytes / time is the streaming bandwidth this GPU sustains, the
 * ceiling the dispatch and combine bandwidths are also reported against,
 * and the plain copy of known size that calibrates HBM byte counters.
 */
moe_status_t moe_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
