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
#include <type_traits>

#include "device_util.h"
#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

constexpr int GROUP_M = 8;  // row tiles per group of the tile order (8 measured best)
constexpr int NUM_XCD = 8;

// Per-expert tile prefix in LDS: s_prefix[e] = sum_{e' < e} ceil(rows_e' / bm),
// s_prefix[E] = total row tiles, and a copy of offsets[0..E] in s_off (so
// that the tile lookups need no second global round trip).  Computed by
// wave 0.
__device__ __forceinline__ void build_tile_prefix(const int32_t* __restrict__ offsets, int E, int bm,
                                                  int* s_prefix, int* s_off) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        // lane owns experts 4*lane .. 4*lane+3; all its loads go out together
        // (clamped indices, no branches), so this costs one round trip
        int o[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) o[i] = offsets[min(lane * 4 + i, E)];
        int c[4];
        int local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = (lane * 4 + i < E) ? (o[i + 1] - o[i] + bm - 1) / bm : 0;
            local += c[i];
        }
        int incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        int run = incl - local;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            if (e < E) {
                s_prefix[e] = run;
                s_off[e] = o[i];
            }
            run += c[i];
        }
        if (lane == 63) s_prefix[E] = incl;
        if (lane == 0) s_off[E] = offsets[E];
    }
    __syncthreads();
}

struct Tile {
    int e;       // expert
    int row0;    // first queue row of the tile
    int row1;    // one past the last valid queue row
    int nt;      // column tile
};

// Row tile and column tile of position pid in the tile order: groups of
// GROUP_M row tiles, each group walked column tile by column tile.
__device__ __forceinline__ Tile tile_of(int pid, const int* s_off, int E, int bm, int n_tiles,
                                        const int* s_prefix) {
    const int total_m = s_prefix[E];
    const int group = pid / (GROUP_M * n_tiles);
    const int first_m = group * GROUP_M;
    const int gsz = min(GROUP_M, total_m - first_m);
    const int local = pid - group * GROUP_M * n_tiles;
    const int mt = first_m + local % gsz;
    Tile t;
    t.nt = local / gsz;
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_prefix[mid] <= mt) lo = mid; else hi = mid;
    }
    t.e = lo;
    t.row0 = s_off[lo] + (mt - s_prefix[lo]) * bm;
    t.row1 = min(t.row0 + bm, s_off[lo + 1]);
    return t;
}

// Split-K plan: the first `full` tiles of the order (a multiple of `slots`,
// the workgroups resident at once) run whole; when the rest would leave most
// workgroup slots idle in a last wave, each of them runs as S K ranges.
// slots = 0: no split.
struct SplitPlan {
    int total, full, S;
};
__device__ __forceinline__ SplitPlan split_plan(int total, int slots, int nk) {
    SplitPlan sp{total, total, 1};
    if (slots > 0) {
        const int r = total % slots;
        const int S = r > 0 ? min(slots / r, min(kSplitMax, nk / kSplitMinSlices)) : 1;
        if (S >= 2) {
            sp.full = total - r;
            sp.S = S;
        }
    }
    return sp;
}

// This workgroup's work: a whole tile (j = -1, K slices [0, nk)) or K slices
// [kb, kb + nkl) of split tile number j / S of the tail, whose partial sums
// go to slot j.  The workgroup id is remapped so that each XCD (workgroups
// are dealt to the 8 XCDs round-robin) walks one contiguous range of the
// whole tiles; the split work comes after every whole tile.
struct Work {
    Tile t;
    int kb, nkl, j;
    int kv = 64;  // weight gradients: valid K rows of the last slice
};
__device__ __forceinline__ bool find_work(const int* s_off, int E, int bm, int n_tiles,
                                          const int* s_prefix, int nk, int slots, Work& w) {
    const SplitPlan sp = split_plan(s_prefix[E] * n_tiles, slots, nk);
    const int hw = blockIdx.x;
    const int per_xcd = (sp.full + NUM_XCD - 1) / NUM_XCD;
    int pid;
    if (hw < per_xcd * NUM_XCD) {
        pid = (hw % NUM_XCD) * per_xcd + hw / NUM_XCD;
        if (pid >= sp.full) return false;
        w.kb = 0;
        w.nkl = nk;
        w.j = -1;
    } else {
        const int j = hw - per_xcd * NUM_XCD;
        if (j >= (sp.total - sp.full) * sp.S) return false;
        pid = sp.full + j / sp.S;
        const int part = j % sp.S;
        w.kb = part * nk / sp.S;
        w.nkl = (part + 1) * nk / sp.S - w.kb;
        w.j = j;
    }
    w.t = tile_of(pid, s_off, E, bm, n_tiles, s_prefix);
    return true;
}

// This workgroup's whole tile (no split); false when it has no work.
__device__ __forceinline__ bool find_tile(const int* s_off, int E, int bm, int n_tiles,
                                          const int* s_prefix, Tile& t) {
    Work w;
    if (!find_work(s_off, E, bm, n_tiles, s_prefix, 1, 0, w)) return false;
    t = w.t;
    return true;
}

// silu(g) * u in fp32 (the fp32 problem: correctly rounded exp and divide).
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// The same for the bf16 problem, whose result is rounded to bf16 (8 bits):
// hardware exp2 and reciprocal (about 1 ulp of fp32 each) are far below that.
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * u * __builtin_amdgcn_rcpf(1.f + e);
}

// sigmoid(u) with the same hardware exp2 and reciprocal.
__device__ __forceinline__ float sigmoid_fast(float u) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-u * 1.4426950408889634f));
}

// ---------------------------------------------------------------------------
// bf16 grouped GEMM on MFMA (v_mfma_f32_32x32x16_bf16)
//
// Tile: 256 queue rows ("activation rows", A) x 256 weight rows (B): in GEMM1
// the 256 weight rows are 128 W_gate rows and the same 128 W_up rows, so the
// tile yields 256 x 128 of h; in GEMM2 they are 256 W_down rows.  Both
// operands are contiguous along K.
//
// 4 waves in 2 x 2.  Wave (wm, wn) owns activation rows wm*128 .. +128 and
// weight rows (GEMM2) wn*128 .. +128, or (GEMM1) gate rows wn*64 .. +64 plus
// the matching up rows.  It keeps 4 x 4 accumulators of 32 x 32 (256 fp32
// per lane).  The MFMA takes the weight fragment as its first operand and the
// activation fragment as its second, so an accumulator holds C^T: each lane
// owns one output row and runs of 4 consecutive output columns, which become
// 8-byte stores, and in GEMM1 the gate and up values of one h element sit in
// the same lane and register of blocks nb and nb + 2.
//
// Operand staging: global_load_lds_dwordx4 copies 16 bytes per lane straight
// into LDS (no register round trip), into a ring of two K slices of 64
// columns: one 128-byte line per row and slice.  Each row of a slice is 8
// 16-byte slots, and the slot that holds chunk c of row r is c ^ ((r >> 1) &
// 7), which spreads the 16-byte fragment reads of 16 consecutive rows over
// all LDS banks.  A slice's fragments (4 K steps x 8 blocks) are read into
// registers at its start, so its LDS stage is free after the first K step and
// the next-but-one slice's loads go out spread over the other three K steps:
// an LDS-bound load is a vector-memory instruction that the wave issues in
// order with its MFMAs, and a burst of them stalls the MFMAs behind it.
// Rows past the end of an expert's queue (or past N) load a clamped valid row
// and their results are never stored.
// ---------------------------------------------------------------------------

// LDS slot of chunk c of tile row r: c ^ slot_swizzle(r).
__device__ __forceinline__ int slot_swizzle(int r) { return (r >> 1) & 7; }

// Weight gradients (512-byte LDS rows of 32 chunks): slot of chunk c of row r
// is c ^ wg_swizzle(r).  The transposing reads of one instruction touch 8
// rows (r & 3 = 0..3, twice) of 64 bytes each; flipping chunk bits 2-3 by
// r & 3 puts rows with different r & 3 on different 16-bank groups.
__device__ __forceinline__ int wg_swizzle(int r) { return (r & 3) << 2; }

// A pointer that is wave-uniform but not provably so to the compiler, moved
// to scalar registers.
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// What a grouped GEMM launch computes (the pipeline is shared):
//   kUp    forward GEMM1: gate and up of the queue rows, SwiGLU epilogue -> h
//   kDown  C = A B^T over the queue rows (forward GEMM2; the backward's dh and dx)
//   kUpBwd the backward's recompute of gate and up, with an epilogue that
//          takes dh and writes du, dv (side by side, [rows, 2f]) and h
//   kWgrad weight gradients: per expert e, C_e[M, N] = sum over the
//          expert's queue rows q of A[q, a_row_off + m] B[q, n], with A and
//          B in queue order ([rows, K] and [rows, N]: K is A's row length
//          here), or one of them token-major (row qtok[q] for queue row q),
//          read through transposing LDS reads, so no transposed copy of
//          either operand is made
constexpr int kUp = 0, kDown = 1, kUpBwd = 2, kWgrad = 3;

// Work of a weight-gradient workgroup: tile (mt, nt) of expert e, K slices of
// the expert's padded queue columns.  All the tiles of one expert read the
// same two operand blocks, so they run on one XCD and share its L2: the
// hardware deals workgroup i to XCD i mod 8, and workgroup i takes place
// i / 8 of that XCD's list, which holds whole experts one after another.
// (Dealing the tiles of every expert over all 8 XCDs made each XCD fetch
// every expert's blocks: the weight-gradient GEMMs took 2.94 instead of
// 2.06 ms at 128 experts of about 2048 rows.)  A tile's cost is its
// expert's row count, so the experts are dealt heaviest first (order[], a
// permutation of the experts by descending count) in a snake order, XCD 0
// to 7 and back, which keeps the XCDs' loads even under a skewed routing.
// Within an expert, groups of GROUP_M row tiles walk the column tiles; with a
// token-major A (dy), whose gathered rows cost more to fetch than the queue-
// order B, groups of GROUP_M column tiles walk the row tiles instead, so that
// the tiles running at once share fewer gathered row blocks (same-box: the
// backward 0.3-0.6 % faster on three layers, unchanged on the fourth).
__host__ __device__ __forceinline__ int wgrad_tiles_per_expert(int M, int N) {
    return ((M + kBM - 1) / kBM) * ((N + kDownCols - 1) / kDownCols);
}
__device__ __forceinline__ bool find_wgrad_work(const int32_t* __restrict__ offsets,
                                                const int32_t* __restrict__ order, int E, int M, int N,
                                                bool group_n, Work& w) {
    const int mtn = (M + kBM - 1) / kBM;
    const int ntn = (N + kDownCols - 1) / kDownCols;
    const int per_e = mtn * ntn;
    const int x = blockIdx.x % NUM_XCD;
    const int place = blockIdx.x / NUM_XCD;
    const int j = place / per_e;  // the XCD's j-th expert
    const int rank = j * NUM_XCD + ((j & 1) ? NUM_XCD - 1 - x : x);
    if (rank >= E) return false;
    const int e = order[rank];
    const int local = place % per_e;
    // (group_n: groups of GROUP_M column tiles walk the row tiles instead)
    const int gm = group_n ? ntn : mtn, go = group_n ? mtn : ntn;
    const int group = local / (GROUP_M * go);
    const int first = group * GROUP_M;
    const int gsz = min(GROUP_M, gm - first);
    const int l2 = local - group * GROUP_M * go;
    const int ig = first + l2 % gsz, io = l2 / gsz;
    const int mt = group_n ? io : ig;
    w.t.e = e;
    w.t.nt = group_n ? ig : io;
    w.t.row0 = mt * kBM;
    w.t.row1 = min(M, w.t.row0 + kBM);
    // (K runs over the expert's queue rows in slices of 64; the rows past
    // its end in the last slice are read but zeroed)
    const int k0 = offsets[e], cnt = offsets[e + 1] - k0;
    w.kb = k0;
    w.nkl = (cnt + 63) / 64;
    w.kv = cnt - 64 * (w.nkl - 1);
    w.j = -1;
    return true;
}

// F8: operands are OCP FP8 E4M3 codes (one byte per element) with per-row
// power-of-two scale exponents: a_exp per activation row (per token of x with
// GATHER, else per queue row), b_exp0 / b_exp1 per weight row of B0 / B1
// (indexed e * N + row).  The MFMA is v_mfma_f32_32x32x64_f8f6f4; the scales
// are applied exactly (ldexp) to the fp32 sums before the epilogue.
// Weight gradients with GATHER: one operand (A, or B when GB) is token-major,
// [T, row length], and queue row q reads its token's row qtok[q] (so neither
// x nor dy is copied into queue order).  kUpBwd: row_scale holds each queue
// row's gate.
template <int MODE, bool GATHER, bool WIDE, bool F8 = false, bool GB = false>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_assign, int topk,
    const int32_t* __restrict__ offsets, int E, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, bf16_t* __restrict__ C, int N, int K, int slots,
    float* __restrict__ part, const bf16_t* __restrict__ aux, bf16_t* __restrict__ C2, int M,
    const int32_t* __restrict__ a_exp = nullptr, const int32_t* __restrict__ b_exp0 = nullptr,
    const int32_t* __restrict__ b_exp1 = nullptr, int a_row_off = 0,
    const int32_t* __restrict__ qtok = nullptr, const float* __restrict__ row_scale = nullptr) {
    constexpr bool GATEUP = MODE == kUp || MODE == kUpBwd;
    constexpr bool WG = MODE == kWgrad;
    static_assert(!F8 || MODE == kUp || MODE == kDown, "fp8 operands: forward GEMMs only");
    constexpr int EB = F8 ? 1 : 2;           // bytes per operand element
    constexpr int TM = 256;                  // activation rows per tile
    constexpr int TN = 256;                  // weight rows per tile
    constexpr int BK = 128 / EB;             // K slice width (one 128-byte line per row)
    constexpr int BN_OUT = GATEUP ? TN / 2 : TN;
    // fp8 GEMM2 (MXS): the activation operand is h, E4M3 codes with one
    // E8M0 scale per 32 columns of a row, which the block-scaled MFMA
    // applies; a slice's scales (4 bytes per row) ride in each stage after
    // the operands, one 4-byte load per lane of one instruction per wave.
    constexpr bool MXS = F8 && MODE == kDown;
    // Weight gradients with a token-major operand (G_A: A, G_B: B): each
    // wave loads the token ids of its 16 rows of a slice into LDS (one
    // 4-byte load per lane, 4 slices ahead of the rows' own loads, a ring of
    // 4 slots), and reads those of the slice it refills at the slice's start.
    constexpr bool WGG = WG && GATHER;
    constexpr bool G_A = WGG && !GB;
    constexpr bool G_B = WGG && GB;
    static_assert(!GB || WGG, "GB selects the gathered operand of a weight gradient");
    constexpr int LA = TM / 32;              // activation loads per wave per slice (8 rows each)
    constexpr int LB = TN / 32;              // weight loads per wave per slice
    constexpr int NL = LA + LB + ((MXS || WGG) ? 1 : 0);
    constexpr int ROWB = 128;                // bytes per row of a slice
    constexpr int SA_BYTES = TM * ROWB;
    constexpr int SC_OFF = (TM + TN) * ROWB;  // (MXS) the scales within a stage
    constexpr int STAGE_BYTES = (TM + TN) * ROWB + (MXS ? TM * 4 : 0);
    constexpr int NR = 8;                    // fragment reads per K step (4 activation, 4 weight)
    constexpr int NM = F8 ? 8 : 16;          // MFMAs per K step (fp8: each twice as long)
    constexpr int KS = 4;                    // K steps per slice (32 bytes of each row per step)
    // GEMM1 issues its activation loads first, GEMM2 its weight loads first
    // (the order that measured faster for each).
    constexpr bool A_FIRST = GATEUP;
    static_assert(2 * STAGE_BYTES <= 160 * 1024, "two stages must fit the 160 KB of LDS");
    static_assert(BK * EB == ROWB, "a slice is one 128-byte line per row");
    static_assert(F8 ? 3 * (LA + LB) <= 2 * (KS - 1) * NM : 3 * (LA + LB) <= (KS - 1) * NM,
                  "the refill spreads one load per 3 MFMAs (fp8: two per 3)");
    constexpr int IDS_OFF = 2 * STAGE_BYTES;  // (WGG) the token-id ring: [slot][wave][64 dwords]
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES + (WGG ? 4 * 4 * 256 : 0)];
    // The tile prefix and offsets tables live in stage 0 until the first load.
    int* const s_prefix = reinterpret_cast<int*>(smem);
    int* const s_off = s_prefix + MOE_MAX_EXPERTS + 1;

    Work work;
    if (WG) {
        // (sorted_assign is the expert order, heaviest first, here)
        // (a token-major A is the gathered side: its tiles are the fewer in
        // each concurrent group)
        if (!find_wgrad_work(offsets, sorted_assign, E, M, N, G_A, work)) return;
    } else {
        build_tile_prefix(offsets, E, TM, s_prefix, s_off);
        const int n_tiles = (N + BN_OUT - 1) / BN_OUT;
        // (GEMM1 never splits: its epilogue is not linear in the partial sums)
        if (!find_work(s_off, E, TM, n_tiles, s_prefix, K / BK, GATEUP ? 0 : slots, work)) return;
        // (K / BK: K slices of 128 bytes, for both element sizes)
    }
    const Tile tile = work.t;
    __syncthreads();  // every lookup is done before the loads overwrite the table

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int n0 = tile.nt * BN_OUT;
    const int lrow = lane >> 3;
    const int lslot = lane & 7;

    // Loads: wave w fills activation rows w*64 .. +64 and weight rows
    // w*64 .. +64 of a stage; load j covers 8 rows, lane -> (row lrow, LDS
    // slot lslot), and the slot receives global chunk lslot ^ swizzle(row).
    // Operand rows are addressed as a uniform base plus 32-bit byte offsets
    // (one expert's weights stay below 4 GiB), except gathered activation
    // rows of an x of 2^31 elements or more (WIDE), which take 64-bit
    // addresses.
    static_assert(GATHER || !WIDE, "only gathered rows need 64-bit addresses");
    const char* a_src[WIDE ? LA : 1];
    uint32_t a_off[WIDE ? 1 : LA];
    const char* const Ab = reinterpret_cast<const char*>(A);
    // bytes per operand row (weight gradients: A's rows of K elements)
    const int64_t RB = static_cast<int64_t>(K) * EB;
    // (the K range [work.kb, work.kb + work.nkl) of 128-byte slices is folded
    // into the bases; a weight-gradient tile starts at its expert's first
    // queue row work.kb, at column a_row_off + its first output row; a
    // token-major operand's rows are found per slice instead)
    const char* const a_base =
        uniform_ptr(WG ? Ab + (G_A ? 0 : static_cast<int64_t>(work.kb) * RB) + (a_row_off + tile.row0) * 2
                       : (GATHER ? Ab : Ab + static_cast<int64_t>(tile.row0) * RB) + work.kb * 128);
    // Weight gradients stage a slice as 64 queue rows x 256 channels of each
    // operand (512-byte LDS rows: the same 32 KB per operand, at the same LDS
    // places as the other modes).  Load j of wave w covers queue rows w*16 +
    // 2j and + 1 (lane -> row lane >> 5, slot lane & 31); slot s of row r
    // holds channel chunk s ^ wg_swizzle(r).  One slice advances 64 rows.
    const int64_t RBB = WG ? static_cast<int64_t>(N) * 2 : RB;  // bytes per B row
    const int64_t a_step = WG ? 64 * RB : 128;
    const int64_t b_step = WG ? 64 * RBB : 128;
    // (weight gradients) byte offset of the lane's 16-byte chunk of row r of
    // a slice, for a channel range starting col_bytes into rows of row_bytes.
    // A range that passes the row's end (M or N not a multiple of 256) reads
    // the row's last chunk instead: those channels' results are never
    // stored, and a token-major operand has no padding past its last row.
    auto wg_chunk = [&](int r, int64_t col_bytes, int64_t row_bytes) {
        int64_t c = ((lane & 31) ^ wg_swizzle(r)) * 16;
        if (WGG && col_bytes + c >= row_bytes) c = row_bytes - 16 - col_bytes;
        return static_cast<uint32_t>(c);
    };
    // (gathered rows need a lookup in sorted_assign: called after the first
    // weight loads are on their way)
    auto setup_a = [&]() {
        if constexpr (WG) {
#pragma unroll
            for (int j = 0; j < LA; ++j) {
                const int r = wave * 16 + 2 * j + (lane >> 5);
                a_off[0 * WIDE + j] = (G_A ? 0u : static_cast<uint32_t>(r) * static_cast<uint32_t>(RB)) +
                                      wg_chunk(r, (a_row_off + tile.row0) * 2, RB);
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < LA; ++j) {
            const int r = wave * 64 + j * 8 + lrow;
            const int chunk = lslot ^ slot_swizzle(r);
            int pos = tile.row0 + r;
            if (pos >= tile.row1) pos = tile.row1 - 1;
            if (WIDE)
                a_src[WIDE ? j : 0] =
                    Ab + static_cast<int64_t>(sorted_assign[pos] / topk) * RB + work.kb * 128 + chunk * 16;
            else if (GATHER)
                a_off[WIDE ? 0 : j] = static_cast<uint32_t>(sorted_assign[pos] / topk) * static_cast<uint32_t>(RB) +
                                      chunk * 16u;
            else
                a_off[WIDE ? 0 : j] = static_cast<uint32_t>(pos - tile.row0) * static_cast<uint32_t>(RB) + chunk * 16u;
        }
    };
    // In GEMM1 the first 128 weight rows are gate rows and the rest up rows,
    // so each wave's rows come from one matrix.
    const int rb0 = wave * (TN / 4);
    const char* const b_base =
        uniform_ptr(reinterpret_cast<const char*>(GATEUP && rb0 >= TN / 2 ? B1 : B0) +
                    (WG ? (G_B ? 0 : static_cast<int64_t>(work.kb) * RBB) + static_cast<int64_t>(n0) * 2
                        : static_cast<int64_t>(tile.e) * N * RB + work.kb * 128));
    uint32_t b_off[LB];
#pragma unroll
    for (int j = 0; j < LB; ++j) {
        if (WG) {
            const int r = wave * 16 + 2 * j + (lane >> 5);
            b_off[j] = (G_B ? 0u : static_cast<uint32_t>(r) * static_cast<uint32_t>(RBB)) +
                       wg_chunk(r, n0 * 2, RBB);
            continue;
        }
        const int r = rb0 + j * 8 + lrow;
        const int chunk = lslot ^ slot_swizzle(r);
        int n = n0 + (GATEUP && r >= TN / 2 ? r - TN / 2 : r);
        if (n >= N) n = N - 1;
        b_off[j] = static_cast<uint32_t>(n) * static_cast<uint32_t>(RB) + chunk * 16u;
    }
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
    const uint32_t lds_a = lds0 + wave * 64 * ROWB;
    const uint32_t lds_b = lds0 + SA_BYTES + rb0 * ROWB;
    // activation load j (< LA) and weight load j (< LB) of slice kt
    // (WGG: gid[j] is the token of load j's row in the slice being loaded)
    uint32_t gid[WGG ? LA : 1] = {};
    static_assert(!WGG || LA == LB, "one token id per load of either operand");
    auto dma_a = [&](int j, int kt) {
        const uint32_t so = static_cast<uint32_t>((kt & 1) * STAGE_BYTES);
        if (WIDE) lds_dma16(a_src[WIDE ? j : 0] + kt * 128, lds_a + so + j * 8 * ROWB);
        else if (G_A)
            lds_dma16_s(a_base, gid[WGG ? j : 0] * static_cast<uint32_t>(RB) + a_off[WIDE ? 0 : j],
                        lds_a + so + j * 8 * ROWB);
        else lds_dma16_s(a_base + kt * a_step, a_off[WIDE ? 0 : j], lds_a + so + j * 8 * ROWB);
    };
    auto dma_b = [&](int j, int kt) {
        const uint32_t so = static_cast<uint32_t>((kt & 1) * STAGE_BYTES);
        if (G_B)
            lds_dma16_s(b_base, gid[WGG ? j : 0] * static_cast<uint32_t>(RBB) + b_off[j], lds_b + so + j * 8 * ROWB);
        else lds_dma16_s(b_base + kt * b_step, b_off[j], lds_b + so + j * 8 * ROWB);
    };
    // (WGG) token ids: lane i of wave w loads the id of row w*16 + 2*(i & 7)
    // + ((i >> 3) & 1) of slice kt (lanes 16..63 repeat lanes 0..15), into
    // dword i of the wave's 256-byte region of ring slot kt & 3; a lane then
    // finds the ids of its loads j = 0..7 (rows w*16 + 2j + (lane >> 5)) as
    // 8 consecutive dwords.  Slices past the last load the last one's ids
    // (the expert's rows end within the padding qtok carries).
    const char* id_base = nullptr;
    uint32_t id_voff = 0;
    if constexpr (WGG) {
        id_base = uniform_ptr(reinterpret_cast<const char*>(qtok) + static_cast<int64_t>(work.kb) * 4);
        id_voff = static_cast<uint32_t>(wave * 16 + 2 * (lane & 7) + ((lane >> 3) & 1)) * 4u;
    }
    auto dma_id = [&](int kt) {
        const int kc = min(kt, work.nkl - 1);
        lds_dma4_s(id_base + static_cast<int64_t>(kc) * 256, id_voff,
                   lds0 + IDS_OFF + static_cast<uint32_t>(((kt & 3) * 4 + wave) * 256));
    };
    auto read_ids = [&](int kt) {
        if constexpr (WGG) {
            const char* const src = smem + IDS_OFF + ((kt & 3) * 4 + wave) * 256 + (lane >> 5) * 32;
            const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(src);
            const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(src + 16);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gid[WGG ? j : 0] = lo[j];
                gid[WGG ? 4 + j : 0] = hi[j];
            }
        }
    };
    // (MXS) the scales: LDS dword w*64 + i of the stage (lane i of wave w)
    // holds tile row ((s & 7) << 5) | (s >> 3), s = w*64 + i, so that the
    // rows wm*128 + mb*32 + l (mb = 0..3) of a lane's fragments are 4
    // consecutive dwords; aux holds the scales slice by slice, [K/128][M
    // queue rows][4 bytes]
    uint32_t sc_off = 0;
    const char* sc_base = nullptr;
    if constexpr (MXS) {
        const int sl = wave * 64 + lane;
        int pos = tile.row0 + (((sl & 7) << 5) | (sl >> 3));
        if (pos >= tile.row1) pos = tile.row1 - 1;
        sc_off = static_cast<uint32_t>(pos) * 4u;
        sc_base = uniform_ptr(reinterpret_cast<const char*>(aux) + static_cast<int64_t>(work.kb) * M * 4);
    }
    auto dma_sc = [&](int kt) {
        const uint32_t so = static_cast<uint32_t>((kt & 1) * STAGE_BYTES);
        lds_dma4_s(sc_base + static_cast<int64_t>(kt) * M * 4, sc_off, lds0 + so + SC_OFF + wave * 256);
    };
    // load q (< NL) of slice kt, in the GEMM's load order (MXS: the scales
    // last)
    auto dma = [&](int q, int kt) {
        if (MXS && q == LA + LB) {
            dma_sc(kt);
            return;
        }
        if (WGG && q == LA + LB) {  // (the ids of the slice two later)
            dma_id(kt + 2);
            return;
        }
        const bool a_op = A_FIRST ? q < LA : q >= LB;
        if (a_op) dma_a(A_FIRST ? q : q - LB, kt);
        else dma_b(A_FIRST ? q - LA : q, kt);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // Fragment reads.  A 32-row block starts at a multiple of 32 rows, so the
    // slot swizzle of the lane's row (lane & 31 within the block) is the same
    // in every block: one byte offset per K step serves all blocks.
    const int khalf = lane >> 5;
    const int l32 = lane & 31;
    uint32_t foff[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) foff[kk] = l32 * ROWB + (((2 * kk + khalf) ^ slot_swizzle(l32)) * 16);
    // Weight gradients: a fragment (32 channels x 16 K values) is two
    // transposing reads (ds_read_b64_tr_b16) of the [K][channel] stage.  In
    // each 16-lane group g (lanes 16g + i), lane i addresses queue row
    // (g >> 1) * 8 + (i >> 2) (and + 4 for the second read) and channels
    // (g & 1) * 16 + 4 (i & 3) .. + 4 of the block, and receives channel
    // (g & 1) * 16 + i at the 4 rows from there: element t of the fragment
    // is K row (g >> 1) * 8 + t of the step (lane mapping checked on gfx950).
    // The swizzle flips bits 2-3 of the chunk, so the block's offset depends
    // on the lane's row: one offset per block (A: 0..3, B: 4..7).
    constexpr int WROWB = 512;  // bytes per LDS row of a weight-gradient slice
    static_assert(SA_BYTES == 64 * WROWB, "64 queue rows of 256 channels per operand and stage");
    uint32_t wofs[WG ? NR : 1];
    if constexpr (WG) {
        const int g = lane >> 4, i = lane & 15, q = (i >> 2) & 3;
        const uint32_t rb = static_cast<uint32_t>(((g >> 1) * 8 + (i >> 2)) * WROWB);
        const int low = (g & 1) * 2 + ((i & 3) >> 1);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            wofs[b] = rb + ((wm * 16 + ((b ^ q) << 2) + low) << 4) + 8 * (i & 1);
            wofs[4 + b] = SA_BYTES + rb + ((wn * 16 + ((b ^ q) << 2) + low) << 4) + 8 * (i & 1);
        }
    }
    const char* const sa_w = smem + wm * 128 * ROWB;
    const char* const sb_w = smem + SA_BYTES;
    auto b_row0 = [&](int nb) {
        if (GATEUP) return (nb >> 1) * (TN / 2) + wn * (TN / 4) + (nb & 1) * 32;
        return wn * (TN / 2) + nb * 32;
    };

    const int nk = work.nkl;
    // Weight gradients: in an expert's last slice the queue rows from work.kv
    // on are not the expert's (the next expert's rows, or padding rows past
    // the last queue row).  Each wave zeroes its own rows among them, in
    // both operands, once its loads of that slice have landed and before
    // the barrier that publishes the slice; then the waits that barrier needs.
    auto zero_tail_rows = [&](int kt) {
        if constexpr (WG) {
            if (kt == nk - 1 && work.kv < 64) {
                char* const st = smem + (kt & 1) * STAGE_BYTES + (lane < 32 ? 0 : SA_BYTES) + (lane & 31) * 16;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int r = wave * 16 + j;
                    if (r >= work.kv) *reinterpret_cast<i32x4_t*>(st + r * WROWB) = i32x4_t{0, 0, 0, 0};
                }
                wait_vmcnt_lgkm0<0>();
            }
        }
    };
    // All fragments of one slice: step kk's activation blocks f[kk][0..3] and
    // weight blocks f[kk][4..7].
    bf16x8_t f[F8 ? 1 : KS][NR];
    // fp8: one MFMA takes 64 K values, 32 bytes of a lane's row: the 16-byte
    // fragments of steps 2s and 2s + 1 read into one register tuple g[s]
    // (both operands are laid out alike, so every product pairs the same K
    // index)
    i32x8_t g[F8 ? 2 : 1][NR];
    auto read_frag = [&](int kk, int i, uint32_t so) {
        if constexpr (WG) {
            typedef short ws4_t __attribute__((ext_vector_type(4)));
            typedef __attribute__((address_space(3))) ws4_t* lds_ws4_t;
            const uint32_t a = lds_addr(smem) + so + wofs[i] + kk * 16 * WROWB;
            const ws4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_ws4_t>(a));
            const ws4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_ws4_t>(a + 4 * WROWB));
            f[kk][i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            return;
        }
        const char* base = i < 4 ? sa_w + so + i * 32 * ROWB : sb_w + so + b_row0(i - 4) * ROWB;
        if constexpr (F8) {
            const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(base + foff[2 * kk]);
            const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(base + foff[2 * kk + 1]);
            g[kk][i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            f[kk][i] = *reinterpret_cast<const bf16x8_t*>(base + foff[kk]);
        }
    };
#define MOE_MFMA_BF16(KK, Q)                                                                    \
    acc[(Q) / 4][(Q) % 4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                           \
        f[KK][4 + (Q) / 4], f[KK][(Q) % 4], acc[(Q) / 4][(Q) % 4], 0, 0, 0)
    // (MXS) this slice's scale dwords of the lane's 4 activation rows,
    // shifted so that byte 2s is the lane's K block of fp8 K step s (lanes
    // 32..63 hold the upper 32 of the step's 64 K values), and the next
    // slice's, read during step 3
    uint32_t scv[MXS ? 4 : 1] = {}, scv_n[MXS ? 4 : 1] = {};
    auto read_sc = [&](uint32_t so, uint32_t* dst) {
        if constexpr (MXS) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + so + SC_OFF + (l32 * 8 + wm * 4) * 4);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) dst[mb] = v[mb] >> (8 * khalf);
        }
    };
    // fp8: step S of a slice runs blocks (S & 1) * 8 .. + 8 of fp8 K step S >> 1
    // (MXS: the h operand scaled by its E8M0 byte 2 (S >> 1), the weights by
    // 2^0 = E8M0 127; their row scales follow after the loop)
#define MOE_MFMA_F8(S, J)                                                                       \
    do {                                                                                        \
        constexpr int i_ = ((S) & 1) * 8;                                                       \
        if constexpr (MXS)                                                                      \
            acc[(i_ + (J)) / 4][(i_ + (J)) % 4] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4( \
                g[(S) >> 1][4 + (i_ + (J)) / 4], g[(S) >> 1][(i_ + (J)) % 4],                     \
                acc[(i_ + (J)) / 4][(i_ + (J)) % 4], 0, 0, 0, 0x7F7F7F7F, 2 * ((S) >> 1),         \
                scv[MXS ? (i_ + (J)) % 4 : 0]);                                                 \
        else                                                                                    \
            acc[(i_ + (J)) / 4][(i_ + (J)) % 4] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4( \
                g[(S) >> 1][4 + (i_ + (J)) / 4], g[(S) >> 1][(i_ + (J)) % 4],                     \
                acc[(i_ + (J)) / 4][(i_ + (J)) % 4], 0, 0, 0, 0, 0, 0);                         \
    } while (0)
#define MOE_MFMA(KK, Q)                                                                         \
    do {                                                                                        \
        if constexpr (F8) MOE_MFMA_F8(KK, Q);                                                   \
        else MOE_MFMA_BF16(KK, Q);                                                              \
    } while (0)

    // Per slice kt (stage kt & 1):
    //   step 0: its MFMAs, with the reads of steps 1..3; then every wave has
    //           read the stage, and a barrier frees it;
    //   steps 1..3: MFMAs, with the loads of slice kt + 2 into the freed
    //           stage spread one per 3 MFMAs (almost two slices to land);
    //           before step 3, the wait for slice kt + 1 and the barrier that
    //           publishes it;
    //   step 3 also reads slice kt + 1's step-0 fragments.
    // Loads complete in issue order, so each wait leaves pending exactly the
    // loads of slice kt + 2 issued before it.
    // (fp8: MFMAs twice as long, half as many: two loads per 3 MFMAs)
    // (MXS: the scale load goes out with the first operand load)
    auto refill = [&](int step, int q, int kt) {  // MFMA q of step 1..3
        const int p = (step - 1) * NM + q;
        constexpr int NOP = LA + LB;  // operand loads
        const bool issue = F8 ? (p % 3 != 2 && p - p / 3 < NOP) : (p % 3 == 0 && p / 3 < NOP);
        if ((MXS || WGG) && p == 0) dma(NOP, kt + 2);
        if (issue) {
            dma(F8 ? p - p / 3 : p / 3, kt + 2);
            // keep each load between its MFMAs (the scheduler would
            // otherwise gather them into a burst)
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // loads issued in steps 1..2
    constexpr int BEFORE3_ = (F8 ? 2 * NM - (2 * NM) / 3 : (2 * NM + 2) / 3) + ((MXS || WGG) ? 1 : 0);
    constexpr int BEFORE3 = BEFORE3_ < NL ? BEFORE3_ : NL;
    // fragments read ahead of a slice: bf16 step 0; fp8 step 0 (a register
    // pair per block, used by the slice's first two quarter steps)
    constexpr int KPRE = 1;
    constexpr int KREAD = F8 ? 2 : KS;  // fragment steps per slice
    // Prologue: the weight rows of slices 0 and 1 go out first (their
    // addresses need no lookup), then the activation rows (see above).
    // Issue order B0 B1 A0 A1: slice 0 has landed when at most the LA loads
    // of A1 are pending.
    // (a weight-gradient tile of an expert with no rows has nk = 0: no loads,
    // and its zero accumulators are stored)
    if (nk > 0 && WGG) {
        // ids of slices 0..3, the queue-order operand's slices 0 and 1, then
        // (once the ids have landed) the token-major operand's
        setup_a();
#pragma unroll
        for (int kt0 = 0; kt0 < 4; ++kt0) dma_id(kt0);
        auto dma_q = [&](int j, int kt0) {
            if (G_A) dma_b(j, kt0);
            else dma_a(j, kt0);
        };
        auto dma_t = [&](int j, int kt0) {
            if (G_A) dma_a(j, kt0);
            else dma_b(j, kt0);
        };
#pragma unroll
        for (int j = 0; j < LA; ++j) dma_q(j, 0);
        if (nk > 1) {
#pragma unroll
            for (int j = 0; j < LA; ++j) dma_q(j, 1);
            wait_vmcnt<2 * LA>();
        } else {
            wait_vmcnt<LA>();
        }
        read_ids(0);
#pragma unroll
        for (int j = 0; j < LA; ++j) dma_t(j, 0);
        if (nk > 1) {
            read_ids(1);
#pragma unroll
            for (int j = 0; j < LA; ++j) dma_t(j, 1);
            wait_vmcnt_lgkm0<LA>();
        } else {
            wait_vmcnt_lgkm0<0>();
            zero_tail_rows(0);
        }
        barrier_lds();
#pragma unroll
        for (int i = 0; i < NR; ++i) read_frag(0, i, 0);
        __builtin_amdgcn_sched_barrier(0);
    } else if (nk > 0) {
#pragma unroll
        for (int j = 0; j < LB; ++j) dma_b(j, 0);
        if (nk > 1) {
#pragma unroll
            for (int j = 0; j < LB; ++j) dma_b(j, 1);
        }
        setup_a();
#pragma unroll
        for (int j = 0; j < LA; ++j) dma_a(j, 0);
        if constexpr (MXS) dma_sc(0);
        if (nk > 1) {
#pragma unroll
            for (int j = 0; j < LA; ++j) dma_a(j, 1);
            if constexpr (MXS) dma_sc(1);
            wait_vmcnt_lgkm0<LA + (MXS ? 1 : 0)>();
        } else {
            wait_vmcnt_lgkm0<0>();
            zero_tail_rows(0);
        }
        barrier_lds();
#pragma unroll
        for (int i = 0; i < NR; ++i) read_frag(0, i, 0);
        read_sc(0, scv);
        __builtin_amdgcn_sched_barrier(0);
    }

    // One slice; MORE (a compile-time flag, so that the refills need no
    // branches) says that slice kt + 2 exists: true for all but the last two.
    auto slice = [&](int kt, auto more_c) {
        constexpr bool MORE = decltype(more_c)::value;
        const uint32_t so = static_cast<uint32_t>((kt & 1) * STAGE_BYTES);
        const uint32_t nso = static_cast<uint32_t>(((kt + 1) & 1) * STAGE_BYTES);
        // step 0: the reads of the remaining steps (bf16: 24 over 16 MFMAs;
        // fp8: 16 over 8; weight gradients: 48 transposing reads over 16)
        {
            // (WGG: the token ids of the slice this one refills, first)
            if (MORE) read_ids(kt + 2);
#pragma unroll
            for (int kk = KPRE; kk < KREAD; ++kk)
#pragma unroll
                for (int i = 0; i < NR; ++i) read_frag(kk, i, so);
#pragma unroll
            for (int q = 0; q < NM; ++q) MOE_MFMA(0, q);
            if (WGG && MORE) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            constexpr int RPM = WG ? 3 : 2;  // LDS reads per MFMA in the first half
#pragma unroll
            for (int i = 0; i < NR; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
            }
#pragma unroll
            for (int i = NR; i < NM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, WG ? 3 : 1, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt_lgkm0<63>();
        barrier_lds();
        // steps 1 and 2
#pragma unroll
        for (int step = 1; step <= 2; ++step) {
#pragma unroll
            for (int q = 0; q < NM; ++q) {
                if (step == 1) MOE_MFMA(1, q);
                else MOE_MFMA(2, q);
                if (MORE) refill(step, q, kt);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (MORE) {
            wait_vmcnt<BEFORE3>();
            barrier_lds();
        } else if (kt + 1 < nk) {
            wait_vmcnt<0>();
            zero_tail_rows(kt + 1);
            barrier_lds();
        }
        // step 3 (after the last slice the reads fetch a stale, in-bounds
        // stage whose values are never used)
#pragma unroll
        for (int q = 0; q < NM; ++q) {
            MOE_MFMA(3, q);
            if (MORE) refill(3, q, kt);
            if (F8) {
                read_frag(0, q, nso);  // two 16-byte reads
                if (MXS && q == 0) read_sc(nso, scv_n);
            } else if ((q & 1) && (q >> 1) < NR) {
                read_frag(0, q >> 1, nso);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MXS) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) scv[mb] = scv_n[mb];
        }
    };
    int kt = 0;
    for (; kt + 2 < nk; ++kt) slice(kt, std::true_type{});
    for (; kt < nk; ++kt) slice(kt, std::false_type{});
#undef MOE_MFMA
#undef MOE_MFMA_F8
#undef MOE_MFMA_BF16

    // fp8: apply the row and column scales, 2^(a_exp[row] + b_exp[col]),
    // exactly (before a split partial is stored, which then sums scaled
    // values: the same result, since the scaling is by a power of two)
    if constexpr (F8) {
        int ea[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            int pos = tile.row0 + wm * 128 + mb * 32 + l32;
            if (pos >= tile.row1) pos = tile.row1 - 1;
            ea[mb] = MXS ? 0 : a_exp[GATHER ? sorted_assign[pos] / topk : pos];
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = GATEUP ? n0 + wn * 64 + (nb & 1) * 32 + 8 * g + 4 * khalf
                                       : n0 + wn * 128 + nb * 32 + 8 * g + 4 * khalf;
                const int32_t* be = (GATEUP && nb >= 2) ? b_exp1 : b_exp0;
                i32x4_t eb = {0, 0, 0, 0};
                if (col < N) eb = *reinterpret_cast<const i32x4_t*>(be + static_cast<int64_t>(tile.e) * N + col);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[nb][mb][4 * g + i] = __builtin_amdgcn_ldexpf(acc[nb][mb][4 * g + i], ea[mb] + eb[i]);
            }
    }

    // A split K range: the fp32 partial sums go to slot work.j, register by
    // register (register r of thread t at (j * 256 + r) * 256 + t).
    if (!GATEUP && work.j >= 0) {
        float* const dst = const_cast<float*>(uniform_ptr(part + static_cast<int64_t>(work.j) * 256 * 256));
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int i = 0; i < 16; ++i) dst[((nb * 4 + mb) * 16 + i) * 256 + tid] = acc[nb][mb][i];
        return;
    }

    // Epilogue through LDS.  Block (nb, mb): lane owns tile row wm*128 +
    // mb*32 + (lane & 31) and, for g = 0..3, the 4 output columns 8g +
    // 4*(lane >> 5) + 0..3 of the block (registers 4g .. 4g+3).  The ring is
    // free once every wave has left the loop: the output tile is staged there
    // row-major, 16-byte chunk ch of row r at chunk ch ^ (r mod CPR), which
    // spreads the 8-byte writes of 32 rows over the banks, and then written
    // out in whole 16-byte chunks, consecutive lanes on consecutive chunks of
    // a row, so that every store instruction covers whole 128-byte lines
    // (8-byte stores into 32 rows each took 5-12 us per tile, measured).
    // The stores are non-temporal (no tile of the launch reads another's
    // output): the expert FFN call measured 1.2-1.6 % faster at f = 768 and
    // 1408, with the operand reads' L2 hit rates unchanged within a point.
    constexpr int OUTC = GATEUP ? TN / 2 : TN;  // output columns of a tile
    constexpr int CPR = OUTC / 8;               // 16-byte chunks per row
    constexpr int ROWO = OUTC * 2;              // bytes per staged row
    static_assert(TM * ROWO <= 2 * STAGE_BYTES, "the staged tile must fit the ring");
    wait_vmcnt_lgkm0<0>();
    barrier_lds();
    // (kUpBwd) the gate of each of the lane's 4 rows
    float rs[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (MODE == kUpBwd) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int pos = tile.row0 + wm * 128 + mb * 32 + l32;
            rs[mb] = pos < tile.row1 ? row_scale[pos] : 0.f;
        }
    }
    // stage the tile's output (h = silu(gate) * up for the gate/up modes, the
    // accumulators otherwise; kUpBwd: g h, the row's gate times h, which the
    // SwiGLU backward has left in the gate block's registers) and store it to
    // out (row stride ldo)
    auto stage_and_store = [&](bf16_t* __restrict__ out, int64_t ldo) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int r = wm * 128 + mb * 32 + l32;
            char* const srow = smem + r * ROWO + khalf * 8;
            const int sw = r & (CPR - 1);
#pragma unroll
            for (int nb = 0; nb < (GATEUP ? 2 : 4); ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint2 o;
                    if (GATEUP) {
                        float v[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // (kUpBwd: the gate block's registers already
                            // hold g h, left there by the SwiGLU backward)
                            if (MODE == kUpBwd) v[i] = acc[nb][mb][4 * g + i];
                            else v[i] = silu_mul_fast(acc[nb][mb][4 * g + i], acc[nb + 2][mb][4 * g + i]);
                        }
                        o = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                    } else {
                        const f32x16_t& a = acc[nb][mb];
                        o = make_uint2(pack_bf16x2(a[4 * g], a[4 * g + 1]), pack_bf16x2(a[4 * g + 2], a[4 * g + 3]));
                    }
                    const int ch = (GATEUP ? wn * 8 : wn * 16) + nb * 4 + g;
                    *reinterpret_cast<uint2*>(srow + ((ch ^ sw) * 16)) = o;
                }
        }
        __syncthreads();
#pragma unroll 4
        for (int idx = tid; idx < TM * CPR; idx += 256) {
            const int r = idx / CPR;
            const int ch = idx % CPR;
            const int pos = tile.row0 + r;
            const int col = n0 + ch * 8;
            if (pos >= tile.row1 || col >= N) continue;
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(smem + r * ROWO + ((ch ^ (r & (CPR - 1))) * 16));
            __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out + static_cast<int64_t>(pos) * ldo + col));
        }
    };

    if constexpr (F8 && GATEUP) {
        // fp8 GEMM1: h = silu(gate) * up rounded to bf16 and quantised for
        // GEMM2 per block of 32 columns of a row: the block's exponent a is
        // the smallest with max|block| <= 448 * 2^a (0 for a zero block), at
        // least -127, stored as the E8M0 byte a + 127, and each value becomes
        // the E4M3 code of value / 2^a (round to nearest even).  A block's 32
        // values sit in lanes l and l + 32 of the wave (16 each).  The codes
        // are staged as 256 rows of 128 bytes (16-byte chunk ch of row r at
        // chunk ch ^ (r & 7)), the 4 scale bytes of each row after them; C
        // receives the codes [M rows, N], C2 the scales, slice by slice
        // ([N / 128][M][4]: tile column nt is GEMM2's K slice nt).
        char* const s_codes = smem;
        unsigned char* const s_sc = reinterpret_cast<unsigned char*>(smem + TM * 128);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int r = wm * 128 + mb * 32 + l32;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                float v[16];
                float am = 0.f;
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const uint32_t w = pack_bf16x2(silu_mul_fast(acc[nb][mb][i], acc[nb + 2][mb][i]),
                                                   silu_mul_fast(acc[nb][mb][i + 1], acc[nb + 2][mb][i + 1]));
                    v[i] = lo_bf16(w);
                    v[i + 1] = hi_bf16(w);
                    am = fmaxf(am, fmaxf(fabsf(v[i]), fabsf(v[i + 1])));
                }
                am = fmaxf(am, __shfl_xor(am, 32, 64));
                // am = mm 2^e with mm in [0.5, 1); 448 = 0.875 * 2^9
                int a = 0;
                if (am > 0.f) {
                    int e = 0;
                    const float mm = frexpf(am, &e);
                    a = mm <= 0.875f ? e - 9 : e - 8;
                }
                a = max(a, -127);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(v[4 * g], -a),
                                                            __builtin_amdgcn_ldexpf(v[4 * g + 1], -a), 0, false);
                    w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(v[4 * g + 2], -a),
                                                        __builtin_amdgcn_ldexpf(v[4 * g + 3], -a), w, true);
                    const int c = wn * 64 + nb * 32 + 8 * g + 4 * khalf;  // byte column of the tile
                    *reinterpret_cast<int*>(s_codes + r * 128 + (((c >> 4) ^ (r & 7)) << 4) + (c & 15)) = w;
                }
                if (khalf == 0) s_sc[r * 4 + wn * 2 + nb] = static_cast<unsigned char>(a + 127);
            }
        }
        __syncthreads();
        unsigned char* const hq = reinterpret_cast<unsigned char*>(C);
#pragma unroll 4
        for (int idx = tid; idx < TM * 8; idx += 256) {
            const int r = idx >> 3;
            const int ch = idx & 7;
            const int pos = tile.row0 + r;
            const int col = n0 + ch * 16;
            if (pos >= tile.row1 || col >= N) continue;
            *reinterpret_cast<uint4*>(hq + static_cast<int64_t>(pos) * N + col) =
                *reinterpret_cast<const uint4*>(s_codes + r * 128 + ((ch ^ (r & 7)) << 4));
        }
        const int pos = tile.row0 + tid;
        if (pos < tile.row1)
            *reinterpret_cast<uint32_t*>(reinterpret_cast<unsigned char*>(C2) +
                                         (static_cast<int64_t>(tile.nt) * M + pos) * 4) =
                *reinterpret_cast<const uint32_t*>(s_sc + tid * 4);
        return;
    }

    if (MODE == kUpBwd) {
        // The backward of SwiGLU from the recomputed gate u and up v and the
        // incoming dh = g dh_raw (aux holds dh_raw = dy W_down, [rows, f];
        // g is the row's gate): with sg = sigmoid(u), s = u sg,
        // du = dh v sg (1 + u (1 - sg)) and dv = dh s.  Pass 1 stages du and
        // dv side by side (a 256-column row: chunks 0..15 du, 16..31 dv) and
        // stores them to C = [rows, 2f] (du in columns [0, f), dv in [f, 2f));
        // pass 2 stores g h = g s v to C2 (the down projection's weight
        // gradient sums dy[t] (g h) over the queue rows).  The gate times
        // the slot gradient's share of the tile's columns, the sum of dv v =
        // g dh_raw s v over them (g <dy[t], y_perm[pos]> = g <dy[t] W_down,
        // h>), goes to part: [rows][2 * column tiles] fp32, one value per
        // wave column half, summed in a fixed order (lane's 32 columns, then
        // lane + 32's).
        constexpr int CPR2 = 32;
        constexpr int ROWO2 = CPR2 * 16;
        static_assert(TM * ROWO2 <= 2 * STAGE_BYTES, "the staged du/dv tile must fit the ring");
        const int ptiles = 2 * ((N + BN_OUT - 1) / BN_OUT);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int r = wm * 128 + mb * 32 + l32;
            const int pos = tile.row0 + r;
            char* const srow = smem + r * ROWO2 + khalf * 8;
            const int sw = r & (CPR2 - 1);
            float dgp = 0.f;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = n0 + wn * 64 + nb * 32 + 8 * g + 4 * khalf;
                    uint2 dhw = make_uint2(0u, 0u);
                    if (pos < tile.row1 && col < N)
                        dhw = *reinterpret_cast<const uint2*>(aux + static_cast<int64_t>(pos) * N + col);
                    const float dr[4] = {lo_bf16(dhw.x), hi_bf16(dhw.x), lo_bf16(dhw.y), hi_bf16(dhw.y)};
                    float du[4], dv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float u = acc[nb][mb][4 * g + i];
                        const float v = acc[nb + 2][mb][4 * g + i];
                        const float sg = sigmoid_fast(u);
                        const float su = u * sg;
                        const float dh = rs[mb] * dr[i];
                        du[i] = dh * v * sg * (1.f + u * (1.f - sg));
                        dv[i] = dh * su;
                        dgp = fmaf(dv[i], v, dgp);
                        // g h for pass 2, in place of u (no second exp)
                        acc[nb][mb][4 * g + i] = rs[mb] * su * v;
                    }
                    const int ch = wn * 8 + nb * 4 + g;
                    *reinterpret_cast<uint2*>(srow + ((ch ^ sw) * 16)) =
                        make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
                    *reinterpret_cast<uint2*>(srow + (((ch + 16) ^ sw) * 16)) =
                        make_uint2(pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3]));
                }
            const float tot = dgp + __shfl_xor(dgp, 32, 64);
            if (khalf == 0 && pos < tile.row1) part[static_cast<int64_t>(pos) * ptiles + tile.nt * 2 + wn] = tot;
        }
        __syncthreads();
#pragma unroll 4
        for (int idx = tid; idx < TM * CPR2; idx += 256) {
            const int r = idx / CPR2;
            const int ch = idx % CPR2;
            const int pos = tile.row0 + r;
            const int col = n0 + (ch & 15) * 8;
            if (pos >= tile.row1 || col >= N) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(smem + r * ROWO2 + ((ch ^ (r & (CPR2 - 1))) * 16));
            *reinterpret_cast<uint4*>(C + static_cast<int64_t>(pos) * (2 * N) + (ch < 16 ? col : N + col)) = v;
        }
        __syncthreads();
        stage_and_store(C2, N);
    } else if (WG) {
        stage_and_store(C + static_cast<int64_t>(tile.e) * M * N, N);
    } else {
        stage_and_store(C, N);
    }
}

// Split-K reduction of the down projection's tail: 16 workgroups per split
// tile t, one per 32 x 32 accumulator block (nb, mb) of each wave, sum the S
// partial tiles in a fixed order (so the result does not depend on
// scheduling) and store the block as the GEMM2 epilogue would.
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part,
                                                           const int32_t* __restrict__ offsets, int E,
                                                           int N, int nk, int slots,
                                                           bf16_t* __restrict__ C) {
    __shared__ int s_prefix[MOE_MAX_EXPERTS + 1];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    build_tile_prefix(offsets, E, kBM, s_prefix, s_off);
    const int n_tiles = (N + kDownCols - 1) / kDownCols;
    const SplitPlan sp = split_plan(s_prefix[E] * n_tiles, slots, nk);
    const int t = blockIdx.x >> 4;
    if (t >= sp.total - sp.full) return;
    const int nb = (blockIdx.x >> 2) & 3;
    const int mb = blockIdx.x & 3;
    const Tile tile = tile_of(sp.full + t, s_off, E, kBM, n_tiles, s_prefix);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int pos = tile.row0 + (wave >> 1) * 128 + mb * 32 + (lane & 31);
    if (pos >= tile.row1) return;
    const int r0 = (nb * 4 + mb) * 16;
    const float* src = part + (static_cast<int64_t>(t) * sp.S * 256 + r0) * 256 + tid;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = src[i * 256];
    for (int sidx = 1; sidx < sp.S; ++sidx) {
        const float* ps = src + static_cast<int64_t>(sidx) * 256 * 256;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] += ps[i * 256];
    }
    bf16_t* crow = C + static_cast<int64_t>(pos) * N;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int col = tile.nt * kDownCols + (wave & 1) * 128 + nb * 32 + 8 * g + 4 * (lane >> 5);
        if (col >= N) continue;
        *reinterpret_cast<uint2*>(crow + col) =
            make_uint2(pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3]));
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
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];

    build_tile_prefix(offsets, E, kF32BM, s_prefix, s_off);
    const int n_tiles = (N + kF32BN - 1) / kF32BN;
    Tile tile;
    if (!find_tile(s_off, E, kF32BM, n_tiles, s_prefix, tile)) return;

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
        return m * std::max(ceil_div(p.f, kGateUpCols), ceil_div(p.d, kDownCols)) + NUM_XCD + kSplitWGs;
    }
    const int64_t m = max_m_tiles(n, p.E, kF32BM);
    return m * std::max(ceil_div(p.f, kF32BN), ceil_div(p.d, kF32BN)) + NUM_XCD;
}

// Workgroups of the bf16 GEMM that run at once on the device of stream s:
// one per CU (each takes 160 KB of LDS), at most kSplitWGs; 0 if unknown.
int resident_slots(hipStream_t s) {
    hipDevice_t dev = 0;
    int cus = 0;
    if (hipStreamGetDevice(s, &dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 0;
    return std::min(cus, kSplitWGs);
}

hipError_t launch_expert_ffn(const moe_problem_t& p, const void* x_perm, const void* x,
                             const int32_t* sorted_assign, const int32_t* offsets,
                             const void* w_gate, const void* w_up, const void* w_down,
                             void* ffn_ws, void* y_perm, hipStream_t s) {
    const int64_t n = p.T * p.k;
    const bool gather = (x_perm == nullptr);
    void* h = ffn_ws;
    if (p.dtype == MOE_DTYPE_BF16) {
        const bf16_t* a = static_cast<const bf16_t*>(gather ? x : x_perm);
        const bf16_t* wg = static_cast<const bf16_t*>(w_gate);
        const bf16_t* wu = static_cast<const bf16_t*>(w_up);
        const bf16_t* wd = static_cast<const bf16_t*>(w_down);
        bf16_t* hb = static_cast<bf16_t*>(h);
        bf16_t* yb = static_cast<bf16_t*>(y_perm);
        // (a gathered x of 2^31 elements or more needs 64-bit row addresses)
        const bool wide = gather && p.T * p.d >= (int64_t{1} << 31);
        // GEMM1 (K = d): gate and up, SwiGLU epilogue -> h
        {
            const unsigned g = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.f, kGateUpCols)));
            if (wide)
                grouped_gemm_bf16_kernel<kUp, true, true><<<g, 256, 0, s>>>(
                    a, sorted_assign, p.k, offsets, p.E, wg, wu, hb, p.f, p.d, 0, nullptr, nullptr, nullptr, 0);
            else if (gather)
                grouped_gemm_bf16_kernel<kUp, true, false><<<g, 256, 0, s>>>(
                    a, sorted_assign, p.k, offsets, p.E, wg, wu, hb, p.f, p.d, 0, nullptr, nullptr, nullptr, 0);
            else
                grouped_gemm_bf16_kernel<kUp, false, false><<<g, 256, 0, s>>>(
                    a, sorted_assign, p.k, offsets, p.E, wg, wu, hb, p.f, p.d, 0, nullptr, nullptr, nullptr, 0);
        }
        // GEMM2 (K = f): down projection -> y_perm, its tail split in K
        {
            const unsigned g = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.d, kDownCols)));
            const int slots = ffn_can_split(p) ? resident_slots(s) : 0;
            float* part =
                slots > 0 ? reinterpret_cast<float*>(static_cast<char*>(ffn_ws) + ffn_h_bytes(p)) : nullptr;
            grouped_gemm_bf16_kernel<kDown, false, false><<<g + (slots > 0 ? kSplitWGs : 0), 256, 0, s>>>(
                hb, sorted_assign, p.k, offsets, p.E, wd, nullptr, yb, p.d, p.f, slots, part, nullptr, nullptr, 0);
            if (slots > 0)
                split_reduce_kernel<<<kSplitWGs * 16, 256, 0, s>>>(part, offsets, p.E, p.d, p.f / 64, slots, yb);
        }
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

// ---- backward GEMMs (bf16) ----------------------------------------------

// dh_raw = dy W_down over the queues, dy's rows gathered by token like x in
// GEMM1 (W_down_t = W_down transposed, [E, f, d]); the gate is applied in the
// recompute's epilogue.
hipError_t launch_backward_dh(const moe_problem_t& p, const void* dy, const int32_t* sorted_assign,
                              const int32_t* offsets, const void* w_down_t, void* dh, hipStream_t s) {
    const int64_t n = p.T * p.k;
    const unsigned g = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.f, kDownCols)));
    // (the backward's limits keep T * d below 2^31: 32-bit gather offsets)
    grouped_gemm_bf16_kernel<kDown, true, false><<<g, 256, 0, s>>>(
        static_cast<const bf16_t*>(dy), sorted_assign, p.k, offsets, p.E,
        static_cast<const bf16_t*>(w_down_t), nullptr, static_cast<bf16_t*>(dh), p.f, p.d, 0, nullptr,
        nullptr, nullptr, 0);
    return hipGetLastError();
}

// Recompute of gate and up from x (gathered), with the SwiGLU backward in the
// epilogue: dh = g dh_raw (qgate: each queue row's gate), du, dv -> duv
// [T*k, 2f], g h -> hg [T*k, f], and the gate-weighted slot gradients'
// partial sums dg_part [T*k][2 ceil(f / 128)] (sum of g dh_raw h over each
// 64 columns).
hipError_t launch_backward_recompute(const moe_problem_t& p, const void* x, const int32_t* sorted_assign,
                                     const int32_t* offsets, const void* w_gate, const void* w_up,
                                     const void* dh, const float* qgate, void* duv, void* hg, float* dg_part,
                                     hipStream_t s) {
    const int64_t n = p.T * p.k;
    const unsigned g = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.f, kGateUpCols)));
    // (the backward's limits keep T * d below 2^31: 32-bit gather offsets)
    grouped_gemm_bf16_kernel<kUpBwd, true, false><<<g, 256, 0, s>>>(
        static_cast<const bf16_t*>(x), sorted_assign, p.k, offsets, p.E, static_cast<const bf16_t*>(w_gate),
        static_cast<const bf16_t*>(w_up), static_cast<bf16_t*>(duv), p.f, p.d, 0, dg_part,
        static_cast<const bf16_t*>(dh), static_cast<bf16_t*>(hg), 0, nullptr, nullptr, nullptr, 0, nullptr,
        qgate);
    return hipGetLastError();
}

// dx_perm = [du dv] [W_gate; W_up] over the queues (W_gu_t = [E, d, 2f]).
// The tail of the tile order splits K as in the forward's down projection
// (part: kSplitWGs partial tiles, or null when bwd_can_split is false).
hipError_t launch_backward_dxperm(const moe_problem_t& p, const void* duv, const int32_t* offsets,
                                  const void* w_gu_t, void* dx_perm, float* part, hipStream_t s) {
    const int64_t n = p.T * p.k;
    const unsigned g = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.d, kDownCols)));
    const int slots = (part != nullptr && bwd_can_split(p)) ? resident_slots(s) : 0;
    grouped_gemm_bf16_kernel<kDown, false, false><<<g + (slots > 0 ? kSplitWGs : 0), 256, 0, s>>>(
        static_cast<const bf16_t*>(duv), nullptr, p.k, offsets, p.E, static_cast<const bf16_t*>(w_gu_t),
        nullptr, static_cast<bf16_t*>(dx_perm), p.d, 2 * p.f, slots, part, nullptr, nullptr, 0);
    if (slots > 0)
        split_reduce_kernel<<<kSplitWGs * 16, 256, 0, s>>>(part, offsets, p.E, p.d, (2 * p.f) / 64, slots,
                                                          static_cast<bf16_t*>(dx_perm));
    return hipGetLastError();
}

// Weight gradient per expert: C[e] [M, N] = sum over the expert's queue rows
// q in [offsets[e], offsets[e+1]) of A[q, a_col_off + m] B[q, n]; order: the
// experts by descending row count.  One operand is token-major (B when
// gather_b, else A): queue row q is its row qtok[q] (qtok carries 64 valid
// entries past the last queue row); the other is in queue order, [rows, lda]
// or [rows, N], with kWgradPadRows rows after the last queue row.
hipError_t launch_backward_wgrad(const moe_problem_t& p, const void* A, int lda, int a_col_off, int M,
                                 const void* B, int N, const int32_t* offsets, const int32_t* order,
                                 const int32_t* qtok, bool gather_b, void* C, hipStream_t s) {
    // (every XCD's list is sized for the most experts one XCD receives)
    const int64_t tiles =
        ceil_div(p.E, NUM_XCD) * NUM_XCD * static_cast<int64_t>(wgrad_tiles_per_expert(M, N));
    const unsigned g = static_cast<unsigned>(tiles);
    // (the backward's limits keep T * d below 2^31: 32-bit row offsets)
    if (gather_b)
        grouped_gemm_bf16_kernel<kWgrad, true, false, false, true><<<g, 256, 0, s>>>(
            static_cast<const bf16_t*>(A), order, p.k, offsets, p.E, static_cast<const bf16_t*>(B), nullptr,
            static_cast<bf16_t*>(C), N, lda, 0, nullptr, nullptr, nullptr, M, nullptr, nullptr, nullptr,
            a_col_off, qtok);
    else
        grouped_gemm_bf16_kernel<kWgrad, true, false, false, false><<<g, 256, 0, s>>>(
            static_cast<const bf16_t*>(A), order, p.k, offsets, p.E, static_cast<const bf16_t*>(B), nullptr,
            static_cast<bf16_t*>(C), N, lda, 0, nullptr, nullptr, nullptr, M, nullptr, nullptr, nullptr,
            a_col_off, qtok);
    return hipGetLastError();
}

// ---- fp8 expert FFN ------------------------------------------------------

// GEMM1 on fp8 codes of x (gathered per queue row) and of W_gate / W_up, with
// the SwiGLU epilogue, writes h as E4M3 codes h_q [T*k, f] with one E8M0
// scale per 32 columns (h_sc, [f / 128][T*k][4] bytes); GEMM2 on the codes of
// h and W_down, on the block-scaled MFMA, writes y_perm.  The down projection
// splits its tail like the bf16 one (part: kSplitWGs partial tiles, or null).
hipError_t launch_expert_ffn_fp8(const moe_problem_t& p, const void* x_q, const int32_t* x_exp,
                                 const int32_t* sorted_assign, const int32_t* offsets, const void* wg_q,
                                 const int32_t* wg_exp, const void* wu_q, const int32_t* wu_exp,
                                 const void* wd_q, const int32_t* wd_exp, void* h_q, void* h_sc, float* part,
                                 void* y_perm, hipStream_t s) {
    const int64_t n = p.T * p.k;
    const int mrows = static_cast<int>(n);  // (queue rows: the scales' row count)
    const unsigned g1 = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.f, kGateUpCols)));
    grouped_gemm_bf16_kernel<kUp, true, false, true><<<g1, 256, 0, s>>>(
        static_cast<const bf16_t*>(x_q), sorted_assign, p.k, offsets, p.E, static_cast<const bf16_t*>(wg_q),
        static_cast<const bf16_t*>(wu_q), static_cast<bf16_t*>(h_q), p.f, p.d, 0, nullptr, nullptr,
        static_cast<bf16_t*>(h_sc), mrows, x_exp, wg_exp, wu_exp);
    const unsigned g2 = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.d, kDownCols)));
    const int nk2 = p.f / 128;
    const int slots = (part != nullptr && fp8_can_split(p)) ? resident_slots(s) : 0;
    grouped_gemm_bf16_kernel<kDown, false, false, true><<<g2 + (slots > 0 ? kSplitWGs : 0), 256, 0, s>>>(
        static_cast<const bf16_t*>(h_q), sorted_assign, p.k, offsets, p.E, static_cast<const bf16_t*>(wd_q),
        nullptr, static_cast<bf16_t*>(y_perm), p.d, p.f, slots, part, static_cast<const bf16_t*>(h_sc), nullptr,
        mrows, nullptr, wd_exp, nullptr);
    if (slots > 0)
        split_reduce_kernel<<<kSplitWGs * 16, 256, 0, s>>>(part, offsets, p.E, p.d, nk2, slots,
                                                          static_cast<bf16_t*>(y_perm));
    return hipGetLastError();
}

}  // namespace moe
