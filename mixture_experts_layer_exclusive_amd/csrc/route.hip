// Router GEMM and static top-k gating.
//
// The router picks a few experts per token (Piper, Japanese explainer,
// opening section); the policy is static top-k (MoEBlaze summary,
// Limitations).  Selection is exact on fp32 logits with ties broken toward
// the lower expert id; gates are the softmax renormalised over the k chosen
// logits.
#include <float.h>
#include <limits.h>

#include "device_util.h"
#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {

namespace {

// ---- router GEMM: logits[T, E] = x[T, d] * W_r[E, d]^T, fp32 accumulate ----
//
// 64 tokens x 64 experts per workgroup, 32-wide reduction chunks staged in
// LDS, 4 x 4 outputs per thread.
constexpr int RT_M = 64;
constexpr int RT_N = 64;
constexpr int RT_K = 32;

template <typename TIn>
__device__ __forceinline__ float load_in(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float load_in<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_in<bf16_t>(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename TIn>
__global__ __launch_bounds__(256) void router_logits_kernel(const TIn* __restrict__ x,
                                                           const TIn* __restrict__ w,
                                                           float* __restrict__ logits,
                                                           int64_t T, int d, int E) {
    __shared__ float xs[RT_K][RT_M + 4];
    __shared__ float ws[RT_K][RT_N + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15;   // expert group
    const int ty = tid >> 4;   // token group
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * RT_M;
    const int e0 = blockIdx.y * RT_N;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

    for (int k0 = 0; k0 < d; k0 += RT_K) {
#pragma unroll
        for (int i = 0; i < (RT_M * RT_K) / 256; ++i) {
            const int idx = tid + 256 * i;
            const int r = idx / RT_K, c = idx % RT_K;
            const int64_t t = t0 + r;
            const int kk = k0 + c;
            xs[c][r] = (t < T && kk < d) ? load_in(x, t * d + kk) : 0.f;
            const int e = e0 + r;
            ws[c][r] = (e < E && kk < d) ? load_in(w, static_cast<int64_t>(e) * d + kk) : 0.f;
        }
        __syncthreads();
#pragma unroll 8
        for (int c = 0; c < RT_K; ++c) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[c][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = ws[c][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = e0 + tx * 4 + j;
            if (e < E) logits[t * E + e] = acc[i][j];
        }
    }
}

// ---- bf16 router GEMM on MFMA, fragments from global memory (E <= 32) -------
//
// A workgroup takes 32 tokens and all experts; its 4 waves split the hidden
// dimension in four.  Each wave computes logits^T blocks of 32 experts x 32
// tokens with v_mfma_f32_32x32x16_bf16, loading its fragments straight from
// global memory (x rows stream from HBM once; the small router weight stays
// in L2).  The partial sums of the four waves are added in LDS in a fixed
// order, so the result does not depend on scheduling.  The kernel is bound by
// the HBM read of x.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int EB>
__global__ __launch_bounds__(256) void router_logits_mfma_kernel(const bf16_t* __restrict__ x,
                                                                const bf16_t* __restrict__ w,
                                                                float* __restrict__ logits,
                                                                int64_t T, int d, int E) {
    __shared__ float part[3][EB][16][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 32;
    int64_t tok = t0 + (lane & 31);
    if (tok >= T) tok = T - 1;  // clamped rows compute discarded outputs
    const int kq = 8 * (lane >> 5);
    const bf16_t* xr = x + tok * d + kq;
    const bf16_t* wr[EB];
#pragma unroll
    for (int b = 0; b < EB; ++b) {
        int e = b * 32 + (lane & 31);
        if (e >= E) e = E - 1;
        wr[b] = w + static_cast<int64_t>(e) * d + kq;
    }
    f32x16_t acc[EB];
#pragma unroll
    for (int b = 0; b < EB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

    const int kspan = d / 4;  // multiple of 16
    const int k1 = (wave + 1) * kspan;
    int k = wave * kspan;
    // 8 K steps per round so that 8 x-row loads are in flight per wave
    for (; k + 128 <= k1; k += 128) {
        bf16x8_t xf[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) xf[s] = *reinterpret_cast<const bf16x8_t*>(xr + k + 16 * s);
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int b = 0; b < EB; ++b) {
                const bf16x8_t wf = *reinterpret_cast<const bf16x8_t*>(wr[b] + k + 16 * s);
                acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf[s], acc[b], 0, 0, 0);
            }
    }
    for (; k < k1; k += 16) {
        const bf16x8_t xf = *reinterpret_cast<const bf16x8_t*>(xr + k);
#pragma unroll
        for (int b = 0; b < EB; ++b) {
            const bf16x8_t wf = *reinterpret_cast<const bf16x8_t*>(wr[b] + k);
            acc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf, acc[b], 0, 0, 0);
        }
    }
    if (wave > 0) {
#pragma unroll
        for (int b = 0; b < EB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) part[wave - 1][b][r][lane] = acc[b][r];
    }
    __syncthreads();
    if (wave != 0) return;
    const int64_t t = t0 + (lane & 31);
    if (t >= T) return;
#pragma unroll
    for (int b = 0; b < EB; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // fixed order: wave 0 + wave 1 + wave 2 + wave 3
            const float v = ((acc[b][r] + part[0][b][r][lane]) + part[1][b][r][lane]) + part[2][b][r][lane];
            // lane holds token (lane & 31); register r holds expert
            // b*32 + 8*(r/4) + 4*(lane/32) + r%4
            const int e = b * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (e < E) logits[t * E + e] = v;
        }
    }
}

// ---- bf16 router GEMM with the operands staged in LDS -----------------------
//
// A workgroup takes 32 TB tokens and all E experts (EB blocks of 32).  Per K
// chunk of 64 columns, the chunk of every router row and of the token
// rows is copied global -> LDS in whole 128-byte lines (global_load_lds,
// 16 bytes per lane, 8 rows per instruction) into a ring of NS stages, so
// the loads of the next NS - 1 chunks are in flight while the MFMAs run on
// the current one.  When EB is a multiple of 4 the waves split the expert
// blocks (wave w: blocks w, w + 4, ...) and each sums over the whole hidden
// dimension; otherwise wave w runs K step w of every chunk and the four
// partial sums are added in LDS in a fixed order.  Both orders are fixed, so
// the logits do not depend on scheduling.  Row r's 16-byte chunk c sits at
// slot c ^ ((r >> 1) & 7) of its 128-byte line, which puts the fragment
// reads of consecutive rows on distinct LDS banks.
//
// TB token blocks of 32 per workgroup (TB = 2 only when the waves split the
// expert blocks): the router rows of a chunk then serve 64 tokens, halving
// their L2 and LDS traffic per token; with 3 stages two such workgroups fit
// a CU's LDS.
template <int EB, int TB = 1, int NS = 4>
__global__ __launch_bounds__(256) void router_logits_lds_kernel(const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ w,
                                                               float* __restrict__ logits, int64_t T,
                                                               int d, int E) {
    constexpr bool SPLIT_E = EB % 4 == 0;
    static_assert(TB == 1 || SPLIT_E, "two token blocks only when the waves split the expert blocks");
    constexpr int NB = SPLIT_E ? EB / 4 : EB;  // expert blocks per wave
    constexpr int ROWS = EB * 32 + 32 * TB;    // router rows, then the token rows
    constexpr int LPW = ROWS / 32;             // load instructions per wave and chunk (8 rows each)
    constexpr int STAGE = ROWS * 128;
    static_assert(NS * STAGE <= 160 * 1024, "the ring must fit the LDS");
    static_assert(SPLIT_E || 3 * EB * 16 * 64 * 4 <= NS * STAGE, "the partial sums reuse the ring");
    __shared__ __attribute__((aligned(1024))) char ring[NS * STAGE];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * (32 * TB);

    // load j of wave w covers rows (w LPW + j) * 8 .. + 8; lane l fills slot
    // l & 7 of row (l >> 3) with the row's global chunk (l & 7) ^ swizzle
    const char* src[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int r = (wave * LPW + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        const bf16_t* row;
        if (r < EB * 32) {
            row = w + static_cast<int64_t>(r < E ? r : E - 1) * d;  // rows past E: discarded outputs
        } else {
            int64_t tok = t0 + (r - EB * 32);
            if (tok >= T) tok = T - 1;                               // clamped tokens: discarded outputs
            row = x + tok * d;
        }
        src[j] = reinterpret_cast<const char*>(row) + c * 16;
    }
    const uint32_t ring0 = __builtin_amdgcn_readfirstlane(lds_addr(ring));
    auto issue = [&](int kc) {
        const uint32_t base = ring0 + (kc % NS) * STAGE + wave * LPW * 8 * 128;
#pragma unroll
        for (int j = 0; j < LPW; ++j) lds_dma16(src[j] + kc * 128, base + j * 8 * 128);
    };
    const int nchunk = d / 64;
#pragma unroll
    for (int c = 0; c < NS - 1; ++c)
        if (c < nchunk) issue(c);

    f32x16_t acc[NB][TB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int u = 0; u < TB; ++u)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[b][u][r] = 0.f;
    // fragment of K step s of a 32-row block starting at row rb: lane l
    // reads row rb + (l & 31), 8 columns from 16 s + 8 (l >> 5)
    const int l32 = lane & 31;
    const int h = lane >> 5;
    auto frag = [&](const char* st, int rb, int s) {
        const int r = rb + l32;
        return *reinterpret_cast<const bf16x8_t*>(st + r * 128 + (((2 * s + h) ^ ((r >> 1) & 7)) * 16));
    };
    for (int kc = 0; kc < nchunk; ++kc) {
        // chunk kc has landed when at most the loads of chunks kc + 1 and
        // kc + 2 are pending; the barrier then publishes it, and every wave
        // is done with chunk kc - 1, whose stage chunk kc + 3 refills
        const int ahead = nchunk - 1 - kc;
        static_assert(NS == 3 || NS == 4, "ring of 3 or 4 stages");
        if (NS == 4 && ahead >= 2) wait_vmcnt_lgkm0<(NS - 2) * LPW>();
        else if (ahead >= 1) wait_vmcnt_lgkm0<LPW>();
        else wait_vmcnt_lgkm0<0>();
        barrier_lds();
        if (kc + NS - 1 < nchunk) issue(kc + NS - 1);
        const char* st = ring + (kc % NS) * STAGE;
        if (SPLIT_E) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8_t xf[TB];
#pragma unroll
                for (int u = 0; u < TB; ++u) xf[u] = frag(st, EB * 32 + 32 * u, s);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const bf16x8_t wf = frag(st, (wave + 4 * b) * 32, s);
#pragma unroll
                    for (int u = 0; u < TB; ++u)
                        acc[b][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf[u], acc[b][u], 0, 0, 0);
                }
            }
        } else {
            const bf16x8_t xf = frag(st, EB * 32, wave);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                acc[b][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(st, b * 32, wave), xf, acc[b][0], 0, 0, 0);
        }
    }

    // lane holds token (lane & 31); register r of block b holds expert
    // 32 b + 8 (r / 4) + 4 (lane / 32) + r % 4
    if (SPLIT_E) {
#pragma unroll
        for (int u = 0; u < TB; ++u) {
            const int64_t tu = t0 + 32 * u + l32;
            if (tu >= T) continue;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int e = (wave + 4 * b) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (e < E) logits[tu * E + e] = acc[b][u][r];
                }
        }
        return;
    }
    const int64_t t = t0 + l32;
    // partial sums of waves 1..3 in the (now idle) ring: [3][EB][16][64]
    float* const part = reinterpret_cast<float*>(ring);
    __syncthreads();
    if (wave > 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) part[(((wave - 1) * EB + b) * 16 + r) * 64 + lane] = acc[b][0][r];
    }
    __syncthreads();
    if (wave != 0 || t >= T) return;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            // fixed order: K step 0 + step 1 + step 2 + step 3
            const float v = ((acc[b][0][r] + part[((0 * EB + b) * 16 + r) * 64 + lane]) +
                             part[((1 * EB + b) * 16 + r) * 64 + lane]) +
                            part[((2 * EB + b) * 16 + r) * 64 + lane];
            const int e = b * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (e < E) logits[t * E + e] = v;
        }
}

// ---- top-k selection and gates: one 64-lane wave per token -----------------
//
// Lane l holds the logits of experts l, l + 64, ... (EPL of them).  Each of
// the k rounds takes every lane's best unchosen (value, id) and reduces it
// across the wave with the order "larger value first, then lower id".  Lane j
// keeps the winner of round j.
__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits,
                                                        int64_t T, int E, int k,
                                                        int32_t* __restrict__ ids,
                                                        float* __restrict__ gates) {
    const int lane = lane_id();
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (t >= T) return;

    float v[EPL];
    bool live[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < E;
        v[i] = live[i] ? logits[t * E + e] : -FLT_MAX;
    }

    float my_v = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -FLT_MAX;
        int be = INT_MAX;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (live[i] && (be == INT_MAX || better(v[i], e, bv, be))) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (oe != INT_MAX && (be == INT_MAX || better(ov, oe, bv, be))) {
                bv = ov;
                be = oe;
            }
        }
        // be is the same on every lane now; its owner retires it.
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + 64 * i == be) live[i] = false;
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
    }

    // gates: softmax over the k chosen logits, shifted by the largest (slot 0)
    const float m = __shfl(my_v, 0, 64);
    const float pj = (lane < k) ? expf(my_v - m) : 0.f;
    float s = pj;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane < k) {
        ids[t * k + lane] = my_e;
        gates[t * k + lane] = pj / s;
    }
}

// ---- top-k for k <= 8: a group of G lanes per token ----------------------
//
// For small k a whole wave per token spends its time in k rounds of 64-lane
// shuffle reductions.  Here G consecutive lanes share a token: lane s of the
// group reads experts 4s .. 4s+3, then 4s + 4G .. (float4 loads when E is a
// multiple of 4, else experts s, s + G, ...), always in ascending id order,
// and keeps the best KM of them as a list sorted by the order "larger value
// first, then lower id".  An expert arriving in ascending id order loses
// every tie against the list, so it is inserted before the first entry it
// strictly exceeds.  The G lists are then merged with xor shuffles; a
// merged-in entry may carry any id, so the merge compares with the full
// order.  The top k of the merged list (k <= KM) is the token's choice,
// identical to k rounds of "take the best remaining expert".
template <int KM>
__device__ __forceinline__ void topk_insert(float v, int e, bool full_order, float (&sv)[KM], int (&se)[KM]) {
    bool c[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) c[j] = v > sv[j] || (full_order && v == sv[j] && e < se[j]);
    // the list is sorted, so c is false ... false true ... true: the entry
    // goes to the first true slot and the ones after it shift down by one
#pragma unroll
    for (int j = KM - 1; j > 0; --j) {
        const float pv = c[j - 1] ? sv[j - 1] : v;
        const int pe = c[j - 1] ? se[j - 1] : e;
        sv[j] = c[j] ? pv : sv[j];
        se[j] = c[j] ? pe : se[j];
    }
    sv[0] = c[0] ? v : sv[0];
    se[0] = c[0] ? e : se[0];
}

template <int KM, int G, int NCH, bool VEC>
__global__ __launch_bounds__(256) void route_topk_group_kernel(const float* __restrict__ logits, int64_t T,
                                                              int E, int k, int32_t* __restrict__ ids,
                                                              float* __restrict__ gates) {
    static_assert(KM >= 1 && KM <= 8 && (G & (G - 1)) == 0 && G <= 64, "group and list sizes");
    const int64_t gt = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t t = gt / G;
    const int s = static_cast<int>(gt % G);
    // lanes past the last token work on a clamped token (every lane of a
    // group takes part in the shuffles) and store nothing
    const float* __restrict__ row = logits + (t < T ? t : T - 1) * static_cast<int64_t>(E);

    float sv[KM];
    int se[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        sv[j] = -INFINITY;  // finite logits always beat the empty slots
        se[j] = INT_MAX;
    }
    if (VEC) {
        // NCH chunks of 4 experts per lane, all loads issued first
        float4 buf[NCH];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int e0 = 4 * (s + c * G);
            buf[c] = e0 < E ? *reinterpret_cast<const float4*>(row + e0) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int e0 = 4 * (s + c * G);
            if (e0 < E) {
                topk_insert<KM>(buf[c].x, e0, false, sv, se);
                topk_insert<KM>(buf[c].y, e0 + 1, false, sv, se);
                topk_insert<KM>(buf[c].z, e0 + 2, false, sv, se);
                topk_insert<KM>(buf[c].w, e0 + 3, false, sv, se);
            }
        }
    } else {
        for (int e = s; e < E; e += G) topk_insert<KM>(row[e], e, false, sv, se);
    }
    // merge the G lists of the group: after round `off`, lanes s and s ^ off
    // hold the same list (the best KM of the union under a total order)
#pragma unroll
    for (int off = 1; off < G; off <<= 1) {
        float ov[KM];
        int oe[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            ov[j] = __shfl_xor(sv[j], off, 64);
            oe[j] = __shfl_xor(se[j], off, 64);
        }
#pragma unroll
        for (int j = 0; j < KM; ++j) topk_insert<KM>(ov[j], oe[j], true, sv, se);
    }
    if (t >= T) return;
    // gates: softmax over the k chosen logits, shifted by the largest (slot 0)
    float p[KM];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        p[j] = j < k ? expf(sv[j] - sv[0]) : 0.f;
        sum += p[j];
    }
#pragma unroll
    for (int j = 0; j < KM; ++j) {
        if (j < k && j % G == s) {
            ids[t * k + j] = se[j];
            gates[t * k + j] = p[j] / sum;
        }
    }
}

}  // namespace

hipError_t launch_router_logits(const moe_problem_t& p, const void* x, const void* w_router,
                                float* logits, hipStream_t s) {
    if (p.dtype == MOE_DTYPE_F32) {
        dim3 grid(static_cast<unsigned>(ceil_div(p.T, RT_M)), static_cast<unsigned>(ceil_div(p.E, RT_N)));
        router_logits_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x),
                                                         static_cast<const float*>(w_router), logits,
                                                         p.T, p.d, p.E);
        return hipGetLastError();
    }
    const unsigned grid = static_cast<unsigned>(ceil_div(p.T, 32));
    // One expert block (E <= 32): fragments straight from global memory are
    // faster (18.5 against 22 us on 8192 x 4096 tokens, 8 experts); more
    // blocks re-read the router rows per token block, and the LDS ring wins
    // (50 against 115 us with top-k, 32768 x 2048 tokens, 128 experts).
    const bool use_lds_router = p.E > 32;
    const unsigned grid2 = static_cast<unsigned>(ceil_div(p.T, 64));  // two token blocks per workgroup
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const bf16_t* wb = static_cast<const bf16_t*>(w_router);
    if (use_lds_router) {
        switch (ceil_div(p.E, 32)) {
            case 2: router_logits_lds_kernel<2><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;  // (E > 32: two blocks or more)
            case 3: router_logits_lds_kernel<3><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
            case 4: router_logits_lds_kernel<4, 2, 3><<<grid2, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
            case 5: router_logits_lds_kernel<5><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
            case 6: router_logits_lds_kernel<6><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
            case 7: router_logits_lds_kernel<7><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
            default: router_logits_lds_kernel<8, 2, 3><<<grid2, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E); break;
        }
        return hipGetLastError();
    }
    router_logits_mfma_kernel<1><<<grid, 256, 0, s>>>(xb, wb, logits, p.T, p.d, p.E);
    return hipGetLastError();
}

hipError_t launch_route_topk(const moe_problem_t& p, const float* logits, int32_t* ids,
                             float* gates, hipStream_t s) {
    if (p.k <= 8) {
        // G = 4 lanes per token; KM = k rounded up to 2, 4 or 8
        constexpr int G = 4;
        const unsigned grid = static_cast<unsigned>(ceil_div(p.T * G, 256));
        const bool vec = p.E % 4 == 0;
        const int nch = static_cast<int>(ceil_div(p.E, 4 * G));  // float4 chunks per lane (E <= 256: <= 16)
#define MOE_TOPK_VEC(KM)                                                                                   \
    do {                                                                                                   \
        if (!vec) route_topk_group_kernel<KM, G, 1, false><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); \
        else if (nch <= 1) route_topk_group_kernel<KM, G, 1, true><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); \
        else if (nch <= 2) route_topk_group_kernel<KM, G, 2, true><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); \
        else if (nch <= 4) route_topk_group_kernel<KM, G, 4, true><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); \
        else if (nch <= 8) route_topk_group_kernel<KM, G, 8, true><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); \
        else route_topk_group_kernel<KM, G, 16, true><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); \
    } while (0)
        if (p.k <= 2) MOE_TOPK_VEC(2);
        else if (p.k <= 4) MOE_TOPK_VEC(4);
        else MOE_TOPK_VEC(8);
#undef MOE_TOPK_VEC
        return hipGetLastError();
    }
    const unsigned grid = static_cast<unsigned>(ceil_div(p.T, 4));
    const int epl = static_cast<int>(ceil_div(p.E, 64));
    switch (epl) {
        case 1: route_topk_kernel<1><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); break;
        case 2: route_topk_kernel<2><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); break;
        case 3: route_topk_kernel<3><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); break;
        default: route_topk_kernel<4><<<grid, 256, 0, s>>>(logits, p.T, p.E, p.k, ids, gates); break;
    }
    return hipGetLastError();
}

}  // namespace moe
