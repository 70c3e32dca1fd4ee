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

#ifndef GEMM_GROUP_M
#define GEMM_GROUP_M 8
#endif
constexpr int GROUP_M = GEMM_GROUP_M;
constexpr int NUM_XCD = 8;

// bf16 GEMM pipeline shape: K slice width, LDS ring depth, slot swizzle.
#ifndef GEMM_BK
#define GEMM_BK 64
#endif
#ifndef GEMM_STAGES
#define GEMM_STAGES 2
#endif
#ifndef GEMM_SWZ
#define GEMM_SWZ 1
#endif

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

// silu(g) * u in fp32 (the fp32 problem: correctly rounded exp and divide).
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// The same for the bf16 problem, whose result is rounded to bf16 (8 bits):
// hardware exp2 and reciprocal (about 1 ulp of fp32 each) are far below that.
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * u * __builtin_amdgcn_rcpf(1.f + e);
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
// into LDS (no register round trip) into an NSTAGE-deep ring of K slices of
// width BK.  Each row of a slice is BK/8 16-byte slots, and the slot that
// holds chunk c of row r is c ^ swz(r), which spreads the 16-byte fragment
// reads of consecutive rows over all LDS banks.  One barrier per K step: it
// publishes slice kt and frees the slot that slice kt + NSTAGE - 1 refills.
// Rows past the end of an expert's queue (or past N) load a clamped valid row
// and their results are never stored.
// ---------------------------------------------------------------------------
typedef uint16_t bf16x4_t __attribute__((ext_vector_type(4)));

template <int BK, int SWZ>
__device__ __forceinline__ int swz(int r) {
    // BK = 64: 8 slots per row; BK = 32: 4 slots per row
    if (BK == 64) return SWZ == 0 ? (r & 7) : ((r >> 1) & 7);
    return SWZ == 0 ? ((r >> 1) & 3) : ((r >> 2) & 3);
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt: vector-memory counter <= N and all LDS reads returned.
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at LDS address lds_base + 16 * i.  Issued as inline assembly so that the
// compiler does not treat every later LDS read as dependent on it; the caller
// orders it with wait_vmcnt and the workgroup barrier.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gptr), "s"(lds_base)
        : "memory");
}

// Workgroup barrier without a memory fence (the LDS traffic it orders is
// waited for explicitly); the empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

template <bool GATEUP, bool GATHER, int BK, int NSTAGE, int SWZ>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void grouped_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ sorted_assign, int topk,
    const int32_t* __restrict__ offsets, int E, const bf16_t* __restrict__ B0,
    const bf16_t* __restrict__ B1, bf16_t* __restrict__ C, int N, int K) {
    constexpr int TM = 256;                 // activation rows (and weight rows) per tile
    constexpr int BN_OUT = GATEUP ? 128 : 256;
    constexpr int CH = BK / 8;              // 16-byte chunks per row
    constexpr int RPI = 64 / CH;            // rows per load instruction
    constexpr int LPW = 64 / RPI;           // load instructions per wave per operand
    constexpr int SLICE = TM * BK;          // bf16 elements per operand slice
    __shared__ __attribute__((aligned(1024))) bf16_t sA[NSTAGE][SLICE];
    __shared__ __attribute__((aligned(1024))) bf16_t sB[NSTAGE][SLICE];
    __shared__ int s_prefix[MOE_MAX_EXPERTS + 1];

    build_tile_prefix(offsets, E, TM, s_prefix);
    const int n_tiles = (N + BN_OUT - 1) / BN_OUT;
    Tile tile;
    if (!find_tile(offsets, E, TM, n_tiles, s_prefix, tile)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int n0 = tile.nt * BN_OUT;
    const int64_t NK = static_cast<int64_t>(N) * K;

    // Per-lane global sources: wave w fills tile rows w*64 .. w*64+63 of both
    // operands; load j covers rows w*64 + j*RPI .. +RPI, lane -> (row, slot).
    const int lrow = lane / CH;
    const int lslot = lane % CH;
    const bf16_t* a_src[LPW];
    const bf16_t* b_src[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int r = wave * 64 + j * RPI + lrow;       // tile row 0..255
        const int chunk = lslot ^ swz<BK, SWZ>(r);      // global chunk for this LDS slot
        int pos = tile.row0 + r;
        if (pos >= tile.row1) pos = tile.row1 - 1;
        const int64_t arow = GATHER ? static_cast<int64_t>(sorted_assign[pos] / topk) : pos;
        a_src[j] = A + arow * K + chunk * 8;
        int n;
        const bf16_t* base;
        if (GATEUP) {
            n = n0 + (r & 127);
            base = (r < 128 ? B0 : B1) + tile.e * NK;
        } else {
            n = n0 + r;
            base = B0 + tile.e * NK;
        }
        if (n >= N) n = N - 1;
        b_src[j] = base + static_cast<int64_t>(n) * K + chunk * 8;
    }

    const uint32_t lds_a0 = __builtin_amdgcn_readfirstlane(lds_addr(&sA[0][wave * 64 * BK]));
    const uint32_t lds_b0 = __builtin_amdgcn_readfirstlane(lds_addr(&sB[0][wave * 64 * BK]));
    // Load q of a slice (q < 2 * LPW).  GEMM1 issues its activation rows
    // first and GEMM2 its weight rows first, the order that measured faster
    // for each (a few percent: the loads of a slice queue behind each other).
    auto dma = [&](int q, int k0, uint32_t boff) {
        const bool a_op = GATEUP ? q < LPW : q >= LPW;
        const int j = q < LPW ? q : q - LPW;
        if (a_op) lds_dma16(a_src[j] + k0, lds_a0 + boff + j * RPI * BK * 2);
        else lds_dma16(b_src[j] + k0, lds_b0 + boff + j * RPI * BK * 2);
    };
    auto load_slice = [&](int kt) {
        const uint32_t boff = static_cast<uint32_t>((kt % NSTAGE) * SLICE * 2);
#pragma unroll
        for (int q = 0; q < 2 * LPW; ++q) dma(q, kt * BK, boff);
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // fragment rows this lane reads
    int brow[4], arow_l[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
        brow[nb] = GATEUP ? ((nb >> 1) * 128 + wn * 64 + (nb & 1) * 32 + (lane & 31))
                          : (wn * 128 + nb * 32 + (lane & 31));
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) arow_l[mb] = wm * 128 + mb * 32 + (lane & 31);
    const int khalf = lane >> 5;

    // LDS element offsets (within a slice) of this lane's fragment rows, per
    // K step kk of the slice
    constexpr int KS = BK / 16;
    int boffs[KS][4], aoffs[KS][4];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const int c = kk * 2 + khalf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            boffs[kk][i] = brow[i] * BK + ((c ^ swz<BK, SWZ>(brow[i])) * 8);
            aoffs[kk][i] = arow_l[i] * BK + ((c ^ swz<BK, SWZ>(arow_l[i])) * 8);
        }
    }

    const int nk = K / BK;
    constexpr int PER = 2 * LPW;  // LDS DMA instructions per slice per wave
    static_assert(2 * LPW == 16, "the interleaved refill assumes 16 DMAs per slice per wave");
    static_assert(KS % 2 == 0, "fragment double buffer needs an even step count");

    // fragments of one K step: 4 weight blocks, 4 activation blocks, two sets
    bf16x8_t fb[2][4], fa[2][4];
#define MOE_READ_FRAGS(SB, SA, KK, SLOT)                                               \
    _Pragma("unroll") for (int i_ = 0; i_ < 4; ++i_) {                                 \
        fb[SLOT][i_] = *reinterpret_cast<const bf16x8_t*>((SB) + boffs[KK][i_]);     \
        fa[SLOT][i_] = *reinterpret_cast<const bf16x8_t*>((SA) + aoffs[KK][i_]);     \
    }
#define MOE_MFMA_STEP(SLOT)                                                            \
    _Pragma("unroll") for (int nb_ = 0; nb_ < 4; ++nb_)                                \
    _Pragma("unroll") for (int mb_ = 0; mb_ < 4; ++mb_)                                \
        acc[nb_][mb_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[SLOT][nb_], fa[SLOT][mb_], \
                                                                acc[nb_][mb_], 0, 0, 0);
    // spread 8 LDS fragment reads over 16 MFMAs
#define MOE_INTERLEAVE()                                                               \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                                 \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                             \
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                             \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                             \
    }

    // Ring of NSTAGE slices.  Slice kt's barrier sits before its last K step:
    // by then every fragment of slice kt is in registers, so the barrier both
    // frees slot kt % NSTAGE for slice kt + NSTAGE and publishes slice kt + 1,
    // whose first fragments are read while the last MFMAs of slice kt run.
#pragma unroll
    for (int s = 0; s < NSTAGE; ++s)
        if (s < nk) load_slice(s);
    if (nk >= NSTAGE) wait_vmcnt_lgkm0<PER * (NSTAGE - 1)>();
    else wait_vmcnt_lgkm0<0>();
    barrier_lds();
    MOE_READ_FRAGS(sB[0], sA[0], 0, 0)
    __builtin_amdgcn_sched_barrier(0);

    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt % NSTAGE;
        const bf16_t* sa = sA[buf];
        const bf16_t* sb = sB[buf];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int cur = kk & 1;
            if (kk + 1 < KS) {
                MOE_READ_FRAGS(sb, sa, kk + 1, cur ^ 1)
                MOE_MFMA_STEP(cur)
                MOE_INTERLEAVE()
            } else {
                if (kt + 1 < nk) {
                    if (kt + NSTAGE <= nk) wait_vmcnt_lgkm0<PER * (NSTAGE - 2)>();
                    else wait_vmcnt_lgkm0<0>();
                    barrier_lds();
                }
                // The last K step of the slice: its 16 MFMAs interleaved with
                // the refill DMAs of slot kt % NSTAGE (slice kt + NSTAGE) and the
                // next slice's first fragment reads (after the last slice these
                // read a stale, in-bounds slot whose values are never used).
                const bool refill = kt + NSTAGE < nk;
                const uint32_t boff_ = static_cast<uint32_t>(buf * SLICE * 2);
                const int k0_ = (kt + NSTAGE) * BK;
                const int nbuf = (kt + 1) % NSTAGE;
                const bf16_t* nsb = sB[nbuf];
                const bf16_t* nsa = sA[nbuf];
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int nb_ = q >> 2, mb_ = q & 3;
                    acc[nb_][mb_] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[cur][nb_], fa[cur][mb_],
                                                                          acc[nb_][mb_], 0, 0, 0);
                    if (refill) dma(q, k0_, boff_);
                    if (q & 1) {
                        const int i_ = q >> 1;
                        if (i_ < 4) fb[cur ^ 1][i_] = *reinterpret_cast<const bf16x8_t*>(nsb + boffs[0][i_]);
                        else fa[cur ^ 1][i_ - 4] = *reinterpret_cast<const bf16x8_t*>(nsa + aoffs[0][i_ - 4]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#undef MOE_READ_FRAGS
#undef MOE_MFMA_STEP
#undef MOE_INTERLEAVE

    // Epilogue.  Block (nb, mb): lane owns output row m = mb*32 + (lane & 31)
    // and, for g = 0..3, columns nb*32 + 8g + 4*(lane >> 5) + 0..3 (registers
    // 4g .. 4g+3).
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int pos = tile.row0 + wm * 128 + mb * 32 + (lane & 31);
        if (pos >= tile.row1) continue;
        bf16_t* crow = C + static_cast<int64_t>(pos) * N;
        if (GATEUP) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = n0 + wn * 64 + nb * 32 + 8 * g + 4 * khalf;
                    if (col >= N) continue;
                    bf16x4_t o;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        o[i] = f32_to_bf16(silu_mul_fast(acc[nb][mb][4 * g + i], acc[nb + 2][mb][4 * g + i]));
                    *reinterpret_cast<bf16x4_t*>(crow + col) = o;
                }
        } else {
#pragma unroll
            for (int nb = 0; nb < 4; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = n0 + wn * 128 + nb * 32 + 8 * g + 4 * khalf;
                    if (col >= N) continue;
                    bf16x4_t o;
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = f32_to_bf16(acc[nb][mb][4 * g + i]);
                    *reinterpret_cast<bf16x4_t*>(crow + col) = o;
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
            grouped_gemm_bf16_kernel<true, true, GEMM_BK, GEMM_STAGES, GEMM_SWZ><<<g1, 256, 0, s>>>(
                a, sorted_assign, p.k, offsets, p.E, static_cast<const bf16_t*>(w_gate),
                static_cast<const bf16_t*>(w_up), static_cast<bf16_t*>(h), p.f, p.d);
        else
            grouped_gemm_bf16_kernel<true, false, GEMM_BK, GEMM_STAGES, GEMM_SWZ><<<g1, 256, 0, s>>>(
                a, sorted_assign, p.k, offsets, p.E, static_cast<const bf16_t*>(w_gate),
                static_cast<const bf16_t*>(w_up), static_cast<bf16_t*>(h), p.f, p.d);
        const unsigned g2 = grid_for(n, p.E, kBM, static_cast<int>(ceil_div(p.d, kDownCols)));
        grouped_gemm_bf16_kernel<false, false, GEMM_BK, GEMM_STAGES, GEMM_SWZ><<<g2, 256, 0, s>>>(
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
