// Dispatch queues: a stable counting sort of the assignments a = t*k + j by
// expert id (MoEBlaze summary, Methodology 1: compact per-expert queues,
// built during the forward pass, in place of a dense token-by-expert
// routing matrix).
//
// Three passes over the int32 ids:
//   1. histogram: workgroup b counts the experts of assignments
//      [b*C, (b+1)*C) with LDS atomics -> block_counts[e][b] (expert-major);
//   2. scan: one workgroup turns block_counts into an exclusive prefix sum in
//      expert-major order.  Entry [e][b] becomes the first queue position of
//      expert e owned by block b; entry [e][0] is offsets[e];
//   3. scatter: each workgroup walks its chunk again in ascending a, 256
//      assignments per round.  Within a wave, lanes holding the same expert
//      are found with log2(E) ballots (one per id bit), the rank is the
//      popcount of lower peers; ranks across the four waves come from a
//      per-round LDS table.  Visiting a in ascending order in every level
//      makes the sort stable.
// Ids outside [0, E) are skipped (their assign_pos is -1).
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_ITEMS = 8;

__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ ids,
                                                           int64_t n, int E, int nblk,
                                                           int32_t* __restrict__ block_counts) {
    __shared__ int h[MOE_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
    __syncthreads();
    const int64_t a0 = static_cast<int64_t>(blockIdx.x) * kDispatchChunk;
    const int64_t a1 = (a0 + kDispatchChunk < n) ? a0 + kDispatchChunk : n;
    for (int64_t a = a0 + threadIdx.x; a < a1; a += 256) {
        const int e = ids[a];
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
        block_counts[static_cast<int64_t>(e) * nblk + blockIdx.x] = h[e];
}

// In-place exclusive scan of block_counts[E * nblk] by a single workgroup,
// then counts[e] and offsets[e] from the scanned table.
__global__ __launch_bounds__(SCAN_THREADS) void dispatch_scan_kernel(int32_t* __restrict__ bc,
                                                                    int E, int nblk,
                                                                    int32_t* __restrict__ counts,
                                                                    int32_t* __restrict__ offsets) {
    __shared__ int wave_sums[SCAN_THREADS / 64];
    __shared__ int carry_s;
    const int tid = threadIdx.x;
    const int lane = lane_id();
    const int wave = tid >> 6;
    const int64_t total = static_cast<int64_t>(E) * nblk;
    if (tid == 0) carry_s = 0;
    __syncthreads();

    for (int64_t base = 0; base < total; base += SCAN_THREADS * SCAN_ITEMS) {
        const int carry = carry_s;
        int v[SCAN_ITEMS];
        int local = 0;
#pragma unroll
        for (int i = 0; i < SCAN_ITEMS; ++i) {
            const int64_t idx = base + static_cast<int64_t>(tid) * SCAN_ITEMS + i;
            v[i] = idx < total ? bc[idx] : 0;
            local += v[i];
        }
        // inclusive wave scan of the per-thread sums
        int incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (lane >= off) incl += o;
        }
        if (lane == 63) wave_sums[wave] = incl;
        __syncthreads();
        int wave_prefix = 0;
        int tile_total = 0;
        for (int w = 0; w < SCAN_THREADS / 64; ++w) {
            const int sw = wave_sums[w];
            if (w < wave) wave_prefix += sw;
            tile_total += sw;
        }
        int run = carry + wave_prefix + incl - local;
#pragma unroll
        for (int i = 0; i < SCAN_ITEMS; ++i) {
            const int64_t idx = base + static_cast<int64_t>(tid) * SCAN_ITEMS + i;
            if (idx < total) bc[idx] = run;
            run += v[i];
        }
        __syncthreads();
        if (tid == 0) carry_s = carry + tile_total;
        __syncthreads();
    }
    const int grand = carry_s;
    for (int e = tid; e < E; e += SCAN_THREADS) {
        const int lo = bc[static_cast<int64_t>(e) * nblk];
        const int hi = (e + 1 < E) ? bc[static_cast<int64_t>(e + 1) * nblk] : grand;
        offsets[e] = lo;
        counts[e] = hi - lo;
    }
    if (tid == 0) offsets[E] = grand;
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids,
                                                              int64_t n, int E, int nbits, int nblk,
                                                              const int32_t* __restrict__ bases,
                                                              int32_t* __restrict__ sorted_assign,
                                                              int32_t* __restrict__ assign_pos) {
    __shared__ int cursor[MOE_MAX_EXPERTS];
    __shared__ int wcnt[4][MOE_MAX_EXPERTS];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    for (int e = tid; e < E; e += 256) {
        cursor[e] = bases[static_cast<int64_t>(e) * nblk + blockIdx.x];
        wcnt[0][e] = wcnt[1][e] = wcnt[2][e] = wcnt[3][e] = 0;
    }
    __syncthreads();
    const int64_t a0 = static_cast<int64_t>(blockIdx.x) * kDispatchChunk;
    const int64_t a1 = (a0 + kDispatchChunk < n) ? a0 + kDispatchChunk : n;
    for (int64_t base = a0; base < a1; base += 256) {
        const int64_t a = base + tid;
        const bool in_range = a < a1;
        const int e = in_range ? ids[a] : -1;
        const bool ok = in_range && static_cast<unsigned>(e) < static_cast<unsigned>(E);
        uint64_t peers = __ballot(ok);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = ok && ((e >> b) & 1);
            const uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        const int rank = __popcll(peers & lanemask_lt());
        if (ok && rank == 0) wcnt[wave][e] = __popcll(peers);
        __syncthreads();
        if (ok) {
            int pos = cursor[e] + rank;
            for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
            sorted_assign[pos] = static_cast<int32_t>(a);
            assign_pos[a] = pos;
        } else if (in_range) {
            assign_pos[a] = -1;
        }
        __syncthreads();
        for (int x = tid; x < E; x += 256) {
            cursor[x] += wcnt[0][x] + wcnt[1][x] + wcnt[2][x] + wcnt[3][x];
            wcnt[0][x] = wcnt[1][x] = wcnt[2][x] = wcnt[3][x] = 0;
        }
        __syncthreads();
    }
}

// x_perm[pos] = x[sorted_assign[pos] / k] for pos < offsets[E]; one
// workgroup per queue row, 16-byte words when the row allows it.
template <typename W>
__global__ __launch_bounds__(256) void gather_rows_kernel(const W* __restrict__ x,
                                                         const int32_t* __restrict__ sorted_assign,
                                                         const int32_t* __restrict__ offsets, int E,
                                                         int k, int64_t words_per_row,
                                                         W* __restrict__ x_perm) {
    const int64_t pos = blockIdx.x;
    if (pos >= offsets[E]) return;
    const int64_t tok = sorted_assign[pos] / k;
    const W* src = x + tok * words_per_row;
    W* dst = x_perm + pos * words_per_row;
    for (int64_t i = threadIdx.x; i < words_per_row; i += 256) dst[i] = load_nt(src + i);
}

int id_bits(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

}  // namespace

hipError_t launch_dispatch_queues(const moe_problem_t& p, const int32_t* ids, int32_t* counts,
                                  int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos,
                                  int32_t* block_counts, hipStream_t s) {
    const int64_t n = p.T * p.k;
    const int nblk = static_cast<int>(dispatch_blocks(n));
    dispatch_hist_kernel<<<nblk, 256, 0, s>>>(ids, n, p.E, nblk, block_counts);
    dispatch_scan_kernel<<<1, SCAN_THREADS, 0, s>>>(block_counts, p.E, nblk, counts, offsets);
    dispatch_scatter_kernel<<<nblk, 256, 0, s>>>(ids, n, p.E, id_bits(p.E), nblk, block_counts,
                                                 sorted_assign, assign_pos);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const moe_problem_t& p, const void* x, const int32_t* sorted_assign,
                              const int32_t* offsets, void* x_perm, hipStream_t s) {
    const int64_t n = p.T * p.k;
    const int64_t row_bytes = static_cast<int64_t>(p.d) * (p.dtype == MOE_DTYPE_F32 ? 4 : 2);
    if (row_bytes % 16 == 0)
        gather_rows_kernel<uint4><<<static_cast<unsigned>(n), 256, 0, s>>>(
            static_cast<const uint4*>(x), sorted_assign, offsets, p.E, p.k, row_bytes / 16,
            static_cast<uint4*>(x_perm));
    else if (row_bytes % 4 == 0)
        gather_rows_kernel<uint32_t><<<static_cast<unsigned>(n), 256, 0, s>>>(
            static_cast<const uint32_t*>(x), sorted_assign, offsets, p.E, p.k, row_bytes / 4,
            static_cast<uint32_t*>(x_perm));
    else
        gather_rows_kernel<uint16_t><<<static_cast<unsigned>(n), 256, 0, s>>>(
            static_cast<const uint16_t*>(x), sorted_assign, offsets, p.E, p.k, row_bytes / 2,
            static_cast<uint16_t*>(x_perm));
    return hipGetLastError();
}

}  // namespace moe
