// Grouped SwiGLU expert FFN over the dispatch queues.
//
// Every expert e owns the queue rows [offsets[e], offsets[e+1]).  Its FFN is
// two tall-and-skinny GEMMs (Piper technical summary, section 1: fine-grained
// MoE gives tall-and-skinny GEMMs and skewed loads):
//   GEMM1: h = silu(X W_gate[e]^T) * (X W_up[e]^T)   (SwiGLU in the epilogue)
//   GEMM2: y_perm = h W_down[e]^T
// X's rows are gathered straight from x through sorted_assign in GEMM1's
// operand loads when no x_perm is given (MoEBlaze summary, Methodology 2:
// dispatch fused with the expert computation).
//
// Tile schedule: each expert contributes ceil(rows_e / BM) row tiles.  Every
// workgroup rebuilds the per-expert tile prefix from `offsets` in LDS (E is at
// most 256) and finds its expert by binary search, so no host round trip and
// no schedule buffer are needed, and empty or tiny experts cost nothing beyond
// their own tiles.  The 1-D grid is sized for the worst case
// (rows/BM + E row tiles); workgroups past the real tile count exit at once.
//
// Launch order: the hardware deals consecutive workgroups round-robin to the
// 8 XCDs.  The workgroup id is remapped so that each XCD walks one contiguous
// range of the tile order, and that order groups GM row tiles per column
// tile, so the weight tile and the activation tiles a workgroup needs are
// mostly already in its XCD's L2.
#include <algorithm>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GROUP_M = 8;
constexpr int NUM_XCD = 8;

// Per-expert tile prefix in LDS: s_prefix[e] = sum_{e' < e} ceil(rows_e' / bm),
// s_prefix[E] = total row tiles.  Computed by wave 0.
__device__ __forceinline__ void build_tile_prefix(const int32_t* __restrict__ offsets, int E, int bm,
                                                  int* s_prefix) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int c[4];
        int local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            c[i] = (e < E) ? (offsets[e + 1] - offsets[e] + bm - 1) / bm : 0;
            local += c[i];
        }
        int incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        int run = incl - local;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            if (e < E) s_prefix[e] = run;
            run += c[i];
        }
        if (lane == 63) s_prefix[E] = incl;
    }
    __syncthreads();
}

struct Tile {
    int e;       // expert
    int row0;    // first queue row of the tile
    int row1;    // one past the last valid queue row
    int nt;      // column tile
};

// Maps this workgroup to a (row tile, column tile) pair; false when it has
// no work.
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int bm,
                                          int n_tiles, const int* s_prefix, Tile& t) {
    const int total_m = s_prefix[E];
    const int total = total_m * n_tiles;
    const int hw = blockIdx.x;
    const int per_xcd = (total + NUM_XCD - 1) / NUM_XCD;
    if (hw >= per_xcd * NUM_XCD) return false;
    const int pid = (hw % NUM_XCD) * per_xcd + hw / NUM_XCD;
    if (pid >= total) return false;
    const int group = pid / (GROUP_M * n_tiles);
    const int first_m = group * GROUP_M;
    const int gsz = min(GROUP_M, total_m - first_m);
    const int local = pid - group * GROUP_M * n_tiles;
    const int mt = first_m + local % gsz;
    t.nt = local / gsz;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_prefix[mid] <= mt) lo = mid; else hi = mid;
    }
    t.e = lo;
    t.row0 = offsets[lo] + (mt - s_prefix[lo]) * bm;
    t.row1 = min(t.row0 + bm, offsets[lo + 1]);
    return true;
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// ---------------------------------------------------------------------------
// bf16 grouped GEMM on MFMA (v_mfma_f32_32x32x16_bf16)
//
// Tile: 128 queue rows x 256 B rows (GEMM1: 128 gate rows + the same 128 up
// rows; GEMM2: 256 W_down rows), K step 64, both operands K-contiguous.
// 4 waves in 2 x 2; a wave owns 64 rows x 128 B rows = 2 x 4 MFMA blocks of
// 32 x 32 (in GEMM1, blocks 0-1 are gate and 2-3 the matching up columns, so
// the SwiGLU pairs sit in the same lane and register).  Operands are staged
// through double-buffered LDS with rows padded by 16 bytes, which makes the
// 16-byte fragment reads of 32 consecutive rows conflict-free.
// ---------------------------------------------------------------------------
constexpr int LDT = kBK + 8;  // padded LDS row, in bf16 elements
constexpr int B_ROWS = 256;

template <bool GATEUP, bool GATHER>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_assign, int topk,
    const int32_t* __restrict__ offsets, int E, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, bf16_t* __restrict__ C, int N, int K) {
    constexpr int BN_OUT = GATEUP ? kGateUpCols : kDownCols;
    __shared__ __attribute__((aligned(16))) bf16_t sA[2][kBM * LDT];
    __shared__ __attribute__((aligned(16))) bf16_t sB[2][B_ROWS * LDT];
    __shared__ int s_prefix[MOE_MAX_EXPERTS + 1];

    build_tile_prefix(offsets, E, kBM, s_prefix);
    const int n_tiles = (N + BN_OUT - 1) / BN_OUT;
    Tile tile;
    if (!find_tile(offsets, E, kBM, n_tiles, s_prefix, tile)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int cc = tid & 7;         // 16-byte column chunk this thread loads
    const int rbase = tid >> 3;     // first row this thread loads (then +32, +64, ...)
    const int n0 = tile.nt * BN_OUT;
    const int64_t NK = static_cast<int64_t>(N) * K;

    // global source rows of this thread's A and B chunks
    const bf16_t* a_src[4];
    bool a_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pos = tile.row0 + rbase + 32 * i;
        a_ok[i] = pos < tile.row1;
        int64_t row = pos;
        if (GATHER) row = a_ok[i] ? sorted_assign[pos] / topk : 0;
        a_src[i] = A + (a_ok[i] ? row : 0) * K + cc * 8;
    }
    const bf16_t* b_src[8];
    bool b_ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = rbase + 32 * i;
        int n;
        const bf16_t* base;
        if (GATEUP) {
            n = n0 + (r & 127);
            base = (r < 128 ? B0 : B1) + tile.e * NK;
        } else {
            n = n0 + r;
            base = B0 + tile.e * NK;
        }
        b_ok[i] = n < N;
        b_src[i] = base + static_cast<int64_t>(b_ok[i] ? n : 0) * K + cc * 8;
    }

    uint4 ra[4], rb[8];
    const uint4 zero = make_uint4(0, 0, 0, 0);
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ra[i] = a_ok[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : zero;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            rb[i] = b_ok[i] ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : zero;
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(&sA[buf][(rbase + 32 * i) * LDT + cc * 8]) = ra[i];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint4*>(&sB[buf][(rbase + 32 * i) * LDT + cc * 8]) = rb[i];
    };

    f32x16_t acc[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.f;

    // LDS rows this lane reads for its fragments
    const int a_row0 = wm * 64 + (lane & 31);
    int b_row[4];
#pragma unroll
    for (int n = 0; n < 4; ++n)
        b_row[n] = GATEUP ? ((n >> 1) * 128 + wn * 64 + (n & 1) * 32 + (lane & 31))
                          : (wn * 128 + n * 32 + (lane & 31));
    const int kq = (lane >> 5) * 8;

    const int nk = K / kBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            bf16x8_t af[2], bfr[4];
#pragma unroll
            for (int m = 0; m < 2; ++m)
                af[m] = *reinterpret_cast<const bf16x8_t*>(&sA[buf][(a_row0 + m * 32) * LDT + kk * 16 + kq]);
#pragma unroll
            for (int n = 0; n < 4; ++n)
                bfr[n] = *reinterpret_cast<const bf16x8_t*>(&sB[buf][b_row[n] * LDT + kk * 16 + kq]);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfr[n], acc[m][n], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
    // of every 32 x 32 block
    const int col_in = lane & 31;
    const int row_q = (lane >> 5) * 4;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int pos = tile.row0 + wm * 64 + m * 32 + (r >> 2) * 8 + row_q + (r & 3);
            if (pos >= tile.row1) continue;
            bf16_t* crow = C + static_cast<int64_t>(pos) * N;
            if (GATEUP) {
#pragma unroll
                for (int n = 0; n < 2; ++n) {
                    const int col = n0 + wn * 64 + n * 32 + col_in;
                    if (col < N) crow[col] = f32_to_bf16(silu_mul(acc[m][n][r], acc[m][n + 2][r]));
                }
            } else {
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    const int col = n0 + wn * 128 + n * 32 + col_in;
                    if (col < N) crow[col] = f32_to_bf16(acc[m][n][r]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// fp32 grouped GEMM on plain FMA (the fp32 problem keeps every product and
// sum in fp32).  64 x 64 output tile, K step 16, 4 x 4 outputs per thread
// (GEMM1 keeps a gate and an up accumulator per output).
// ---------------------------------------------------------------------------
constexpr int F_BK = 16;

template <bool GATEUP, bool GATHER>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ sorted_assign, int topk,
    const int32_t* __restrict__ offsets, int E, const float* __restrict__ B0,
    const float* __restrict__ B1, float* __restrict__ C, int N, int K) {
    __shared__ float sA[F_BK][kF32BM + 4];
    __shared__ float sB0[F_BK][kF32BN + 4];
    __shared__ float sB1[GATEUP ? F_BK : 1][kF32BN + 4];
    __shared__ int s_prefix[MOE_MAX_EXPERTS + 1];

    build_tile_prefix(offsets, E, kF32BM, s_prefix);
    const int n_tiles = (N + kF32BN - 1) / kF32BN;
    Tile tile;
    if (!find_tile(offsets, E, kF32BM, n_tiles, s_prefix, tile)) return;

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int n0 = tile.nt * kF32BN;
    const int64_t NK = static_cast<int64_t>(N) * K;

    // rows of A this thread loads: r = (tid + 256 i) / 16, column (tid % 16)
    const float* a_src[4];
    bool a_ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = (tid + 256 * i) / F_BK;
        const int pos = tile.row0 + r;
        a_ok[i] = pos < tile.row1;
        int64_t row = pos;
        if (GATHER) row = a_ok[i] ? sorted_assign[pos] / topk : 0;
        a_src[i] = A + (a_ok[i] ? row : 0) * K;
    }
    const int lc = tid % F_BK;

    float acc0[4][4], acc1[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc0[i][j] = acc1[i][j] = 0.f;

    for (int k0 = 0; k0 < K; k0 += F_BK) {
        const int kk = k0 + lc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid + 256 * i) / F_BK;
            sA[lc][r] = (a_ok[i] && kk < K) ? a_src[i][kk] : 0.f;
            const int n = n0 + r;
            const bool bok = n < N && kk < K;
            sB0[lc][r] = bok ? B0[tile.e * NK + static_cast<int64_t>(n) * K + kk] : 0.f;
            if (GATEUP) sB1[lc][r] = bok ? B1[tile.e * NK + static_cast<int64_t>(n) * K + kk] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < F_BK; ++c) {
            float a[4], b0[4], b1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sA[c][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b0[j] = sB0[c][tx * 4 + j];
                if (GATEUP) b1[j] = sB1[c][tx * 4 + j];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc0[i][j] = fmaf(a[i], b0[j], acc0[i][j]);
                    if (GATEUP) acc1[i][j] = fmaf(a[i], b1[j], acc1[i][j]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int pos = tile.row0 + ty * 4 + i;
        if (pos >= tile.row1) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            C[static_cast<int64_t>(pos) * N + n] = GATEUP ? silu_mul(acc0[i][j], acc1[i][j]) : acc0[i][j];
        }
    }
}

unsigned grid_for(int64_t n_rows, int E, int bm, int n_tiles) {
    const int64_t g = max_m_tiles(n_rows, E, bm) * n_tiles;
    return static_cast<unsigned>(align_up(static_cast<size_t>(g), NUM_XCD));
}

}  // namespace

int64_t expert_ffn_grid_bound(const moe_problem_t& p) {
    const int64_t n = p.T * p.k;
    if (p.dtype == MOE_DTYPE_BF16) {
        const int64_t m = max_m_tiles(n, p.E, kBM);
        return m * std::max(ceil_div(p.f, kGateUpCols), ceil_div(p.d, kDownCols)) + NUM_XCD;
    }
    const int64_t m = max_m_tiles(n, p.E, kF32BM);
    return m * std::max(ceil_div(p.f, kF32BN), ceil_div(p.d, kF32BN)) + NUM_XCD;
}

hipError_t launch_expert_ffn(const moe_problem_t& p, const void* x_perm, const void* x,
                             const int32_t* sorted_assign, const int32_t* offsets,
                             const void* w_gate, const void* w_up, const void* w_down,
                             void* h, void* y_perm, hipStream_t s) {
    const int64_t n = p.T * p.k;
    const bool gather = (x_perm == nullptr);
    if (p.dtype == MOE_DTYPE_BF16) {
        const bf16_t* a = static_cast<const bf16_t*>(gather ? x : x_perm);
        const unsigned g1 = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.f, kGateUpCols)));
        if (gather)
            grouped_gemm_bf16_kernel<true, true><<<g1, 256, 0, s>>>(
                a, sorted_assign, p.k, offsets, p.E, static_cast<const bf16_t*>(w_gate),
                static_cast<const bf16_t*>(w_up), static_cast<bf16_t*>(h), p.f, p.d);
        else
            grouped_gemm_bf16_kernel<true, false><<<g1, 256, 0, s>>>(
                a, sorted_assign, p.k, offsets, p.E, static_cast<const bf16_t*>(w_gate),
                static_cast<const bf16_t*>(w_up), static_cast<bf16_t*>(h), p.f, p.d);
        const unsigned g2 = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.d, kDownCols)));
        grouped_gemm_bf16_kernel<false, false><<<g2, 256, 0, s>>>(
            static_cast<const bf16_t*>(h), sorted_assign, p.k, offsets, p.E,
            static_cast<const bf16_t*>(w_down), nullptr, static_cast<bf16_t*>(y_perm), p.d, p.f);
    } else {
        const float* a = static_cast<const float*>(gather ? x : x_perm);
        const unsigned g1 = grid_for(n, p.E, kF32BM, static_cast<int>(ceil_div(p.f, kF32BN)));
        if (gather)
            grouped_gemm_f32_kernel<true, true><<<g1, 256, 0, s>>>(
                a, sorted_assign, p.k, offsets, p.E, static_cast<const float*>(w_gate),
                static_cast<const float*>(w_up), static_cast<float*>(h), p.f, p.d);
        else
            grouped_gemm_f32_kernel<true, false><<<g1, 256, 0, s>>>(
                a, sorted_assign, p.k, offsets, p.E, static_cast<const float*>(w_gate),
                static_cast<const float*>(w_up), static_cast<float*>(h), p.f, p.d);
        const unsigned g2 = grid_for(n, p.E, kF32BM, static_cast<int>(ceil_div(p.d, kF32BN)));
        grouped_gemm_f32_kernel<false, false><<<g2, 256, 0, s>>>(
            static_cast<const float*>(h), sorted_assign, p.k, offsets, p.E,
            static_cast<const float*>(w_down), nullptr, static_cast<float*>(y_perm), p.d, p.f);
    }
    return hipGetLastError();
}

}  // namespace moe
