// Dispatch queues: a stable counting sort of the assignments a = t*k + j by
// expert id (MoEBlaze summary, Methodology 1: compact per-expert queues,
// built during the forward pass, in place of a dense token-by-expert
// routing matrix).
//
// Two passes over the int32 ids:
//   1. histogram: workgroup b counts the experts of assignments
//      [b*C, (b+1)*C) with LDS atomics -> block_counts[e][b] (expert-major);
//      C is a multiple of 256 chosen so that about 256 workgroups run;
//   2. scatter: each workgroup first reduces the expert-major table itself
//      (no separate scan pass): the first queue position of expert e owned by
//      block b is the count of all experts below e plus the counts of e in
//      blocks below b; workgroup 0 also writes counts and offsets.  Then each
//      wave owns a contiguous part of the chunk, counts it, takes its first
//      position per expert from the block base plus the earlier waves'
//      counts, and walks its part in ascending a, 64 at a time: lanes holding
//      the same expert are found with log2(E) ballots (one per id bit) and
//      ranked by the popcount of lower peers.  Ascending a at every level
//      makes the sort stable.
// Up to 4096 assignments both passes run in one 1024-thread workgroup.
// The scatter stages its chunk's ids in LDS first (one bulk load).
// With x_perm, the rows follow in token order (gather_rows_kernel); for
// chunks of 256 ids and a block-count table of at most 4096 entries the
// scatter and the gather are one pass (dispatch_fused_gather_kernel).
// Ids outside [0, E) are skipped (their assign_pos is -1).
#include <algorithm>

#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

// Bits needed for an expert id.
__host__ __device__ __forceinline__ int id_bits(int E) {
    int b = 0;
    while ((1 << b) < E) ++b;
    return b;
}

// Stable ranks of one 64-lane step of a wave's assignments: lanes holding
// the same expert are found with one ballot per id bit; the rank of a lane
// is the number of lower lanes in its group, `count` the group size.
__device__ __forceinline__ void wave_peer_rank(bool ok, int e, int nbits, int& rank, int& count) {
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = ok && ((e >> b) & 1);
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    rank = __popcll(peers & lanemask_lt());
    count = __popcll(peers);
}

// Copies ids[a0 + i], i < cnt (cnt >= 1), into s_ids (LDS), NT threads with
// 8 loads each in flight per round: the load indices are clamped rather than
// guarded, so no branch sits between the loads (a guarded load per element
// made every element a separate round trip to memory).
template <int NT>
__device__ __forceinline__ void stage_ids(const int32_t* __restrict__ ids, int64_t a0, int cnt, int* s_ids) {
    constexpr int U = 8;
    for (int r0 = 0; r0 < cnt; r0 += U * NT) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ids[a0 + min(r0 + u * NT + static_cast<int>(threadIdx.x), cnt - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = r0 + u * NT + static_cast<int>(threadIdx.x);
            if (i < cnt) s_ids[i] = v[u];
        }
    }
}

__global__ __launch_bounds__(256) void dispatch_hist_kernel(const int32_t* __restrict__ ids,
                                                           int64_t n, int64_t chunk, int E, int nblk,
                                                           int32_t* __restrict__ block_counts) {
    __shared__ int h[MOE_MAX_EXPERTS];
    __shared__ int s_ids[kMaxDispatchChunk];
    for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
    const int64_t a0 = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t a1 = (a0 + chunk < n) ? a0 + chunk : n;
    stage_ids<256>(ids, a0, static_cast<int>(a1 - a0), s_ids);
    __syncthreads();
    const int nbits = id_bits(E);
    // one LDS atomic per distinct expert of each 64-lane step (no same-address
    // conflicts inside an instruction)
    for (int64_t base = a0 + (threadIdx.x & ~63); base < a1; base += 256) {
        const int64_t a = base + (threadIdx.x & 63);
        const int e = a < a1 ? s_ids[a - a0] : -1;
        const bool ok = a < a1 && static_cast<unsigned>(e) < static_cast<unsigned>(E);
        int rank, count;
        wave_peer_rank(ok, e, nbits, rank, count);
        if (ok && rank == 0) atomicAdd(&h[e], count);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256)
        block_counts[static_cast<int64_t>(e) * nblk + blockIdx.x] = h[e];
}

// Scatters the assignments [a0, a1) whose experts start at block_base[e]
// (LDS, E entries) in ascending a; s_ids holds their ids (LDS, staged by the
// caller).  NW waves: wave w owns the contiguous sub-range w of the chunk,
// counts it, then walks it 64 at a time with its own LDS cursors, so only two
// workgroup barriers are needed.
template <int NW>
__device__ __forceinline__ void scatter_chunk(const int* s_ids, int64_t a0, int64_t a1,
                                              int E, int nbits, const int* block_base,
                                              int (*wcur)[MOE_MAX_EXPERTS],
                                              int32_t* __restrict__ sorted_assign,
                                              int32_t* __restrict__ assign_pos) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t span = ((a1 - a0) + NW - 1) / NW;
    const int64_t w0 = a0 + wave * span;
    const int64_t w1 = (w0 + span < a1) ? w0 + span : a1;
    // phase 1: per-wave histograms
    for (int x = tid; x < NW * E; x += NW * 64) wcur[x / E][x % E] = 0;
    __syncthreads();
    for (int64_t base = w0; base < w1; base += 64) {
        const int64_t a = base + lane;
        const int e = a < w1 ? s_ids[a - a0] : -1;
        const bool ok = a < w1 && static_cast<unsigned>(e) < static_cast<unsigned>(E);
        int rank, count;
        wave_peer_rank(ok, e, nbits, rank, count);
        if (ok && rank == 0) atomicAdd(&wcur[wave][e], count);
    }
    __syncthreads();
    // phase 2: each wave's first position per expert
    for (int e = tid; e < E; e += NW * 64) {
        int run = block_base[e];
        for (int w = 0; w < NW; ++w) {
            const int c = wcur[w][e];
            wcur[w][e] = run;
            run += c;
        }
    }
    __syncthreads();
    // phase 3: ordered walk, wave-private cursors
    for (int64_t base = w0; base < w1; base += 64) {
        const int64_t a = base + lane;
        const bool in_range = a < w1;
        const int e = in_range ? s_ids[a - a0] : -1;
        const bool ok = in_range && static_cast<unsigned>(e) < static_cast<unsigned>(E);
        int rank, count;
        wave_peer_rank(ok, e, nbits, rank, count);
        int pos = 0;
        if (ok) pos = wcur[wave][e] + rank;
        __builtin_amdgcn_wave_barrier();
        if (ok && rank == 0) wcur[wave][e] += count;
        __builtin_amdgcn_wave_barrier();
        if (ok) {
            sorted_assign[pos] = static_cast<int32_t>(a);
            assign_pos[a] = pos;
        } else if (in_range) {
            assign_pos[a] = -1;
        }
    }
}

// Block b's first queue position per expert, from the expert-major block
// counts bc[E][nblk]: base[e] = sum over experts e' < e of their totals plus
// the counts of e in blocks below b.  Each wave reduces BR expert rows at a
// time (lanes stride over the blocks, so every load is coalesced), with the
// loads of all BR rows in flight together: one row at a time made this a
// chain of E / 4 round trips, the larger part of the scatter at 128 experts.
// Then one wave scans the E totals.  Workgroup 0 also writes counts[E] and
// offsets[E+1].
__device__ __forceinline__ void block_bases(const int32_t* __restrict__ bc, int E, int nblk, int b,
                                            int* s_base, int* s_tot, int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets) {
    constexpr int BR = 8;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int e0 = wave * BR; e0 < E; e0 += 4 * BR) {
        int tot[BR], pre[BR];
#pragma unroll
        for (int r = 0; r < BR; ++r) tot[r] = pre[r] = 0;
#pragma unroll 4
        for (int i = lane; i < nblk; i += 64) {
            int v[BR];
#pragma unroll
            for (int r = 0; r < BR; ++r) v[r] = e0 + r < E ? bc[static_cast<int64_t>(e0 + r) * nblk + i] : 0;
#pragma unroll
            for (int r = 0; r < BR; ++r) {
                tot[r] += v[r];
                pre[r] += i < b ? v[r] : 0;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
#pragma unroll
            for (int r = 0; r < BR; ++r) {
                tot[r] += __shfl_xor(tot[r], off, 64);
                pre[r] += __shfl_xor(pre[r], off, 64);
            }
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < BR; ++r)
                if (e0 + r < E) {
                    s_tot[e0 + r] = tot[r];
                    s_base[e0 + r] = pre[r];
                }
        }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
        int c[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane * 4 + i;
            c[i] = e < E ? s_tot[e] : 0;
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
            if (e < E) {
                s_base[e] += run;
                if (b == 0) {
                    offsets[e] = run;
                    counts[e] = c[i];
                }
            }
            run += c[i];
        }
        if (b == 0 && lane == 63) offsets[E] = incl;
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const int32_t* __restrict__ ids,
                                                              int64_t n, int64_t chunk, int E, int nbits,
                                                              int nblk,
                                                              const int32_t* __restrict__ block_counts,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_assign,
                                                              int32_t* __restrict__ assign_pos) {
    __shared__ int block_base[MOE_MAX_EXPERTS];
    __shared__ int wcur[4][MOE_MAX_EXPERTS];
    __shared__ int s_ids[kMaxDispatchChunk];
    const int64_t a0 = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t a1 = (a0 + chunk < n) ? a0 + chunk : n;
    const int cnt = static_cast<int>(a1 - a0);
    // the first 8 * 256 ids are loaded into registers before the block-count
    // table, so the two round trips to memory overlap; they reach LDS after
    // the table is reduced
    constexpr int U = 8;
    int v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ids[a0 + min(u * 256 + static_cast<int>(threadIdx.x), cnt - 1)];
    // (wcur[0] doubles as the totals' scratch until the scatter clears it)
    block_bases(block_counts, E, nblk, static_cast<int>(blockIdx.x), block_base, wcur[0], counts,
                offsets);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = u * 256 + static_cast<int>(threadIdx.x);
        if (i < cnt) s_ids[i] = v[u];
    }
    if (cnt > U * 256) stage_ids<256>(ids, a0 + U * 256, cnt - U * 256, s_ids + U * 256);
    __syncthreads();
    scatter_chunk<4>(s_ids, a0, a1, E, nbits, block_base, wcur, sorted_assign, assign_pos);
}

// The whole counting sort in one 1024-thread workgroup, for problems small
// enough that one launch beats three: histogram in LDS, exclusive scan over
// the experts, then the ordered scatter.
// (at 16384 assignments the one workgroup took 26 us against 12 us for the
// two launches, cold, measured: one CU does all of the scatter)
constexpr int SMALL_SORT_MAX = 4096;

__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t* __restrict__ ids,
                                                             int64_t n, int E, int nbits,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_assign,
                                                             int32_t* __restrict__ assign_pos) {
    __shared__ int hist[MOE_MAX_EXPERTS];
    __shared__ int base[MOE_MAX_EXPERTS];
    __shared__ int wcur[16][MOE_MAX_EXPERTS];
    __shared__ int s_ids[SMALL_SORT_MAX];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 1024) hist[e] = 0;
    stage_ids<1024>(ids, 0, static_cast<int>(n), s_ids);
    __syncthreads();
    for (int64_t base = tid & ~63; base < n; base += 1024) {
        const int64_t a = base + (tid & 63);
        const int e = a < n ? s_ids[a] : -1;
        const bool ok = a < n && static_cast<unsigned>(e) < static_cast<unsigned>(E);
        int rank, count;
        wave_peer_rank(ok, e, nbits, rank, count);
        if (ok && rank == 0) atomicAdd(&hist[e], count);
    }
    __syncthreads();
    if (tid < 64) {
        // exclusive scan over E <= 256 experts: 4 per lane
        int c[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid * 4 + i;
            c[i] = e < E ? hist[e] : 0;
            local += c[i];
        }
        int incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (tid >= off) incl += o;
        }
        int run = incl - local;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid * 4 + i;
            if (e < E) {
                base[e] = run;
                offsets[e] = run;
                counts[e] = c[i];
            }
            run += c[i];
        }
        if (tid == 63) offsets[E] = incl;
    }
    __syncthreads();
    scatter_chunk<16>(s_ids, 0, n, E, nbits, base, wcur, sorted_assign, assign_pos);
}

// Dispatch gather, token-major: every row of x is read once and written to
// its k queue rows, x_perm[assign_pos[t*k + j]] = x[t] (assignments with no
// queue position are skipped).  A workgroup copies TPB whole rows; threads
// stride over (row, word) pairs, so both the reads and the row writes are
// contiguous, and each thread has U loads in flight before its stores.
template <typename W, int U>
__global__ __launch_bounds__(256) void gather_rows_kernel(const W* __restrict__ x,
                                                         const int32_t* __restrict__ assign_pos,
                                                         int64_t T, int k, int64_t words_per_row,
                                                         int tpb, W* __restrict__ x_perm) {
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
    const int64_t nt = (t0 + tpb <= T) ? tpb : T - t0;
    const int64_t total = nt * words_per_row;
    const W* src = x + t0 * words_per_row;
    for (int64_t i0 = threadIdx.x; i0 < total; i0 += 256 * U) {
        W v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + u * 256;
            if (i < total) v[u] = load_nt(src + i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + u * 256;
            if (i >= total) break;
            const int64_t t = t0 + i / words_per_row;
            const int64_t w = i % words_per_row;
            for (int j = 0; j < k; ++j) {
                const int pos = assign_pos[t * k + j];
                if (pos >= 0) x_perm[static_cast<int64_t>(pos) * words_per_row + w] = v[u];
            }
        }
    }
}

// Scatter and gather in one pass, for small problems with x_perm: chunks of
// 256 assignments and an expert-major block-count table of at most
// kFusedMaxTable entries (written by dispatch_hist_kernel).  Each workgroup
// copies the rows of TPB tokens as gather_rows_kernel does, and first works
// out the queue positions of their assignments itself, by the scatter's own
// rule: pos(a) = offsets[e] + (count of e in the blocks below a's block) +
// (count of e at a' < a in a's block), e = ids[a].  Its row loads are issued
// before the table is read, so the copy's memory latency overlaps the
// position work; it writes sorted_assign and assign_pos for its assignments,
// workgroup 0 also counts and offsets.  Every workgroup reduces the whole
// table (E x blocks entries, from L2).
constexpr int kFusedMaxTable = 4096;
constexpr int kFusedChunk = 256;
// assignments per workgroup: at most one chunk, so they lie in at most two
// consecutive blocks (b_lo and b_lo + 1)
constexpr int kFusedMaxAssign = kFusedChunk;

template <int U>
__global__ __launch_bounds__(256) void dispatch_fused_gather_kernel(
    const int32_t* __restrict__ ids, int E, int k, int nblk, const int32_t* __restrict__ block_counts,
    const uint4* __restrict__ x, int64_t T, int64_t words_per_row, int tpb, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos,
    uint4* __restrict__ x_perm) {
    __shared__ int s_off[MOE_MAX_EXPERTS];     // offsets, then offsets + counts below block b_lo
    __shared__ int s_off1[MOE_MAX_EXPERTS];    // ... below block b_lo + 1
    __shared__ int s_ids[kFusedChunk + kFusedMaxAssign];
    __shared__ int s_pos[kFusedMaxAssign];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * tpb;
    const int64_t nt = (t0 + tpb <= T) ? tpb : T - t0;
    const int64_t total = nt * words_per_row;
    const uint4* src = x + t0 * words_per_row;
    // the first pass of row loads, before anything else
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t i = tid + u * 256;
        if (i < total) v[u] = load_nt(src + i);
    }
    const int64_t a_lo = t0 * k;
    const int m = static_cast<int>(nt * k);
    const int b_lo = static_cast<int>(a_lo / kFusedChunk);
    const int64_t cs = static_cast<int64_t>(b_lo) * kFusedChunk;
    const int nid = static_cast<int>(a_lo + m - cs);
    for (int i = tid; i < nid; i += 256) s_ids[i] = ids[cs + i];
    // per expert (one thread each): its total and its counts below blocks
    // b_lo and b_lo + 1
    int tot = 0, pre0 = 0, pre1 = 0;
    if (tid < E) {
        const int32_t* row = block_counts + static_cast<int64_t>(tid) * nblk;
#pragma unroll 8
        for (int b = 0; b < nblk; ++b) {
            const int c = row[b];
            tot += c;
            pre0 += b < b_lo ? c : 0;
            pre1 += b <= b_lo ? c : 0;
        }
        s_off[tid] = tot;
    }
    __syncthreads();
    if (tid < 64) {
        // exclusive scan of the totals over E <= 256 experts, 4 per lane
        int c[4], local = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid * 4 + i;
            c[i] = e < E ? s_off[e] : 0;
            local += c[i];
        }
        int incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(incl, off, 64);
            if (tid >= off) incl += o;
        }
        int run = incl - local;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = tid * 4 + i;
            if (e < E) {
                s_off1[e] = run;  // (offsets, for now)
                if (blockIdx.x == 0) {
                    offsets[e] = run;
                    counts[e] = c[i];
                }
            }
            run += c[i];
        }
        if (blockIdx.x == 0 && tid == 63) offsets[E] = incl;
    }
    __syncthreads();
    if (tid < E) {
        const int o = s_off1[tid];
        s_off[tid] = o + pre0;
        s_off1[tid] = o + pre1;
    }
    __syncthreads();
    // positions: wave w takes assignments w, w + 4, ...; its lanes count the
    // matching ids below a in a's block 64 at a time
    for (int i = wave; i < m; i += 4) {
        const int64_t a = a_lo + i;
        const int e = s_ids[a - cs];
        int pos = -1;
        if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) {
            const int64_t start = (a / kFusedChunk) * kFusedChunk;
            int rank = 0;
            for (int64_t j0 = start; j0 < a; j0 += 64) {
                const int64_t j = j0 + lane;
                rank += __popcll(__ballot(j < a && s_ids[j - cs] == e));
            }
            pos = (start == cs ? s_off[e] : s_off1[e]) + rank;
        }
        if (lane == 0) {
            s_pos[i] = pos;
            assign_pos[a] = pos;
            if (pos >= 0) sorted_assign[pos] = static_cast<int32_t>(a);
        }
    }
    __syncthreads();
    for (int64_t i0 = tid; i0 < total; i0 += 256 * U) {
        if (i0 != tid) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + u * 256;
                if (i < total) v[u] = load_nt(src + i);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = i0 + u * 256;
            if (i >= total) break;
            const int64_t tl = i / words_per_row;
            const int64_t w = i % words_per_row;
            for (int j = 0; j < k; ++j) {
                const int pos = s_pos[tl * k + j];
                if (pos >= 0) x_perm[static_cast<int64_t>(pos) * words_per_row + w] = v[u];
            }
        }
    }
}

}  // namespace

hipError_t launch_dispatch_queues(const moe_problem_t& p, const int32_t* ids, int32_t* counts,
                                  int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos,
                                  int32_t* block_counts, hipStream_t s) {
    const int64_t n = p.T * p.k;
    if (n <= SMALL_SORT_MAX) {
        dispatch_small_kernel<<<1, 1024, 0, s>>>(ids, n, p.E, id_bits(p.E), counts, offsets,
                                                 sorted_assign, assign_pos);
        return hipGetLastError();
    }
    const int64_t chunk = dispatch_chunk(n);
    const int nblk = static_cast<int>(dispatch_blocks(n));
    dispatch_hist_kernel<<<nblk, 256, 0, s>>>(ids, n, chunk, p.E, nblk, block_counts);
    dispatch_scatter_kernel<<<nblk, 256, 0, s>>>(ids, n, chunk, p.E, id_bits(p.E), nblk, block_counts,
                                                 counts, offsets, sorted_assign, assign_pos);
    return hipGetLastError();
}

hipError_t launch_dispatch(const moe_problem_t& p, const int32_t* ids, const void* x, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, int32_t* block_counts,
                           void* x_perm, hipStream_t s) {
    const int64_t n = p.T * p.k;
    const int64_t row_bytes = static_cast<int64_t>(p.d) * (p.dtype == MOE_DTYPE_F32 ? 4 : 2);
    if (x_perm != nullptr && n > SMALL_SORT_MAX && dispatch_chunk(n) == kFusedChunk &&
        static_cast<int64_t>(p.E) * dispatch_blocks(n) <= kFusedMaxTable && row_bytes % 16 == 0) {
        const int nblk = static_cast<int>(dispatch_blocks(n));
        dispatch_hist_kernel<<<nblk, 256, 0, s>>>(ids, n, kFusedChunk, p.E, nblk, block_counts);
        // rows per workgroup as in the gather (about 32 KB), at most
        // kFusedMaxAssign assignments
        int tpb = static_cast<int>(row_bytes >= 32768 ? 1 : 32768 / row_bytes);
        tpb = std::max(1, std::min(tpb, kFusedMaxAssign / p.k));
        const unsigned grid = static_cast<unsigned>(ceil_div(p.T, tpb));
        dispatch_fused_gather_kernel<8><<<grid, 256, 0, s>>>(
            ids, p.E, p.k, nblk, block_counts, static_cast<const uint4*>(x), p.T, row_bytes / 16, tpb, counts,
            offsets, sorted_assign, assign_pos, static_cast<uint4*>(x_perm));
        return hipGetLastError();
    }
    const hipError_t e = launch_dispatch_queues(p, ids, counts, offsets, sorted_assign, assign_pos, block_counts, s);
    if (e != hipSuccess || x_perm == nullptr) return e;
    return launch_gather_rows(p, x, assign_pos, x_perm, s);
}

hipError_t launch_gather_rows(const moe_problem_t& p, const void* x, const int32_t* assign_pos,
                              void* x_perm, hipStream_t s) {
    const int64_t row_bytes = static_cast<int64_t>(p.d) * (p.dtype == MOE_DTYPE_F32 ? 4 : 2);
    // rows per workgroup: about 32 KB of row data per workgroup (one pass
    // of 256 threads x 8 loads of 16 bytes)
    const int tpb = static_cast<int>(row_bytes >= 32768 ? 1 : 32768 / row_bytes);
    const unsigned grid = static_cast<unsigned>(ceil_div(p.T, tpb));
    if (row_bytes % 16 == 0)
        gather_rows_kernel<uint4, 8><<<grid, 256, 0, s>>>(static_cast<const uint4*>(x), assign_pos, p.T,
                                                      p.k, row_bytes / 16, tpb,
                                                      static_cast<uint4*>(x_perm));
    else if (row_bytes % 4 == 0)
        gather_rows_kernel<uint32_t, 8><<<grid, 256, 0, s>>>(static_cast<const uint32_t*>(x), assign_pos,
                                                         p.T, p.k, row_bytes / 4, tpb,
                                                         static_cast<uint32_t*>(x_perm));
    else
        gather_rows_kernel<uint16_t, 8><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), assign_pos,
                                                         p.T, p.k, row_bytes / 2, tpb,
                                                         static_cast<uint16_t*>(x_perm));
    return hipGetLastError();
}

}  // namespace moe
