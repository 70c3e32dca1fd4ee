// Internal declarations of the MoE-layer HIP library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---- tuning constants --------------------------------------------------------


// bf16 grouped GEMM: queue rows per tile, output columns per tile.
constexpr int kBM = 256;
constexpr int kGateUpCols = 128;  // f-columns per GEMM1 tile (gate and up each)
constexpr int kDownCols = 256;    // output columns per GEMM2 tile

// f32 grouped GEMM tile.
constexpr int kF32BM = 64;
constexpr int kF32BN = 64;

// Split-K of the down projection's last partial wave (bf16): the tiles that
// would leave most CUs idle in a last wave are each cut into S K ranges
// (2 <= S <= kSplitMax, at least kSplitMinSlices 64-wide K slices each) and
// reduced by a second kernel.  The workspace holds kSplitWGs partial tiles.
constexpr int kSplitWGs = 256;
constexpr int kSplitMax = 8;
constexpr int kSplitMinSlices = 8;

// A kernel launch counts its work-items (workgroups x threads) per grid
// dimension in 32 bits.
constexpr int64_t kMaxLaunchItems = 0xffffffffLL;

// ---- small host helpers ------------------------------------------------------

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Expert-FFN workspace: h [T*k, f], then (bf16, when the down projection can
// split) the fp32 partial tiles of the split-K tail.
inline size_t ffn_h_bytes(const moe_problem_t& p) {
    return align_up(static_cast<size_t>(p.T) * p.k * p.f * (p.dtype == MOE_DTYPE_F32 ? 4 : 2), 256);
}
inline bool ffn_can_split(const moe_problem_t& p) {
    return p.dtype == MOE_DTYPE_BF16 && p.f / 64 >= 2 * kSplitMinSlices;
}
inline size_t ffn_split_bytes(const moe_problem_t& p) {
    return ffn_can_split(p) ? static_cast<size_t>(kSplitWGs) * kBM * kDownCols * 4 : 0;
}

// Assignments per workgroup of the histogram and scatter kernels: a multiple
// of 256 sized so that about 256 workgroups (one per CU) share the work, at
// most kMaxDispatchChunk (the scatter stages its chunk's ids in LDS).
constexpr int kMaxDispatchChunk = 8192;
inline int64_t dispatch_chunk(int64_t n_assign) {
    const int64_t c = ceil_div(ceil_div(n_assign, 256), 256) * 256;
    return c < 256 ? 256 : (c > kMaxDispatchChunk ? kMaxDispatchChunk : c);
}
inline int64_t dispatch_blocks(int64_t n_assign) { return ceil_div(n_assign, dispatch_chunk(n_assign)); }

// Upper bound of sum_e ceil(count_e / bm) over any routing of n rows to E experts.
inline int64_t max_m_tiles(int64_t n_rows, int E, int bm) { return n_rows / bm + E; }

// Largest 1-D grid, in 256-thread workgroups, the expert FFN launches for
// problem p (validated against the launch limit before any launch).
int64_t expert_ffn_grid_bound(const moe_problem_t& p);

// ---- launchers (return the launch status) ------------------------------------

hipError_t launch_router_logits(const moe_problem_t& p, const void* x, const void* w_router,
                                float* logits, hipStream_t s);
hipError_t launch_route_topk(const moe_problem_t& p, const float* logits, int32_t* ids,
                             float* gates, hipStream_t s);

hipError_t launch_dispatch_queues(const moe_problem_t& p, const int32_t* ids, int32_t* counts,
                                  int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos,
                                  int32_t* block_counts, hipStream_t s);
// The dispatch: queues, and with x_perm the rows gathered into queue order
// (small problems: one pass does the scatter and the gather).
hipError_t launch_dispatch(const moe_problem_t& p, const int32_t* ids, const void* x, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, int32_t* block_counts,
                           void* x_perm, hipStream_t s);
hipError_t launch_gather_rows(const moe_problem_t& p, const void* x, const int32_t* assign_pos,
                              void* x_perm, hipStream_t s);

hipError_t launch_expert_ffn(const moe_problem_t& p, const void* x_perm, const void* x,
                             const int32_t* sorted_assign, const int32_t* offsets,
                             const void* w_gate, const void* w_up, const void* w_down,
                             void* ffn_ws, void* y_perm, hipStream_t s);

hipError_t launch_combine(const moe_problem_t& p, const void* y_perm, const int32_t* assign_pos,
                          const float* gates, void* y, hipStream_t s);

// ---- backward (bf16) ------------------------------------------------------

// Padded per-expert column count of the weight-gradient operands: every
// expert's queue rounded up to 64 columns.
// The fp8 down projection (K = f codes, 128 per slice) splits its tail too.
inline bool fp8_can_split(const moe_problem_t& p) { return p.f / 128 >= 2 * kSplitMinSlices; }
inline size_t fp8_split_bytes(const moe_problem_t& p) {
    return fp8_can_split(p) ? static_cast<size_t>(kSplitWGs) * kBM * kDownCols * 4 : 0;
}
// The backward's dx_perm GEMM (K = 2f) splits its tail like the down projection.
inline bool bwd_can_split(const moe_problem_t& p) { return (2 * p.f) / 64 >= 2 * kSplitMinSlices; }
inline size_t bwd_split_bytes(const moe_problem_t& p) {
    return bwd_can_split(p) ? static_cast<size_t>(kSplitWGs) * kBM * kDownCols * 4 : 0;
}
// Extra rows after each queue-order operand of the weight-gradient GEMMs: a
// tile reads whole 64-row slices, up to 63 rows past an expert's last row
// (those values are zeroed after the read), plus one row for the channel
// range of a tile that passes a row's end.
constexpr int64_t kWgradPadRows = 65;
inline int64_t backward_kpad(const moe_problem_t& p) {
    return static_cast<int64_t>(align_up(static_cast<size_t>(p.T * p.k + 63 * static_cast<int64_t>(p.E)), 64));
}

hipError_t launch_mfma_peak(int workgroups, int iters, float* sink, hipStream_t s);
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
hipError_t launch_quant_rows_fp8(const void* src, int64_t rows, int cols, void* codes, int32_t* exps,
                                 hipStream_t s);
hipError_t launch_expert_ffn_fp8(const moe_problem_t& p, const void* x_q, const int32_t* x_exp,
                                 const int32_t* sorted_assign, const int32_t* offsets, const void* wg_q,
                                 const int32_t* wg_exp, const void* wu_q, const int32_t* wu_exp,
                                 const void* wd_q, const int32_t* wd_exp, void* h_q, void* h_sc, float* part,
                                 void* y_perm, hipStream_t s);
hipError_t launch_backward_weights(const moe_problem_t& p, const void* w_gate, const void* w_up,
                                   const void* w_down, void* w_down_t, void* w_gu_t, hipStream_t s);
// Slot-gradient partial sums per queue row: one per 64 columns of f (two per
// recompute tile).
inline int bwd_dg_parts(const moe_problem_t& p) { return 2 * static_cast<int>(ceil_div(p.f, kGateUpCols)); }
hipError_t launch_backward_rows(const moe_problem_t& p, const int32_t* assign_pos, const float* gates,
                                int32_t* qtok, float* qgate, hipStream_t s);
hipError_t launch_backward_dl(const moe_problem_t& p, const float* dg_part, const int32_t* ids,
                              const float* gates, const int32_t* assign_pos, float* dsel, float* dlogits,
                              hipStream_t s);
hipError_t launch_backward_poff(const moe_problem_t& p, const int32_t* offsets, int32_t* poff,
                                int32_t* order, int32_t* qtok, hipStream_t s);
hipError_t launch_backward_router_partials(const moe_problem_t& p, const void* x, const int32_t* offsets,
                                           const int32_t* poff, const int32_t* sorted_assign, int64_t kpad,
                                           const float* dsel, float* wr_part, hipStream_t s);
hipError_t launch_backward_dx(const moe_problem_t& p, const void* dx_perm, const int32_t* assign_pos,
                              const int32_t* ids, const float* dsel, const void* w_router, void* dx,
                              hipStream_t s);
hipError_t launch_backward_dwr(const moe_problem_t& p, const float* wr_part, const int32_t* poff,
                               void* dw_router, hipStream_t s);
hipError_t launch_backward_dh(const moe_problem_t& p, const void* dy, const int32_t* sorted_assign,
                              const int32_t* offsets, const void* w_down_t, void* dh, hipStream_t s);
hipError_t launch_backward_recompute(const moe_problem_t& p, const void* x, const int32_t* sorted_assign,
                                     const int32_t* offsets, const void* w_gate, const void* w_up,
                                     const void* dh, const float* qgate, void* duv, void* hg, float* dg_part,
                                     hipStream_t s);
hipError_t launch_backward_dxperm(const moe_problem_t& p, const void* duv, const int32_t* offsets,
                                  const void* w_gu_t, void* dx_perm, float* part, hipStream_t s);
hipError_t launch_backward_wgrad(const moe_problem_t& p, const void* A, int lda, int a_col_off, int M,
                                 const void* B, int N, const int32_t* offsets, const int32_t* order,
                                 const int32_t* qtok, bool gather_b, void* C, hipStream_t s);

}  // namespace moe
