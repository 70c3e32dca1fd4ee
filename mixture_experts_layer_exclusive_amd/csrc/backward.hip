// Backward of the MoE layer, apart from its grouped GEMMs (expert_ffn.hip).
//
// The MoEBlaze summary (euno.news, "MoEBlaze: breaking the memory wall for
// efficient MoE training on modern GPUs"), Methodology item 2, has the
// backward run on the forward's compact dispatch queues; the checkpoint
// bullet of the same item (and Key contributions, bullet 3) recomputes
// intermediates instead of storing them: here the SwiGLU ones.  Here:
//   1. per token: slot gradients dg = <dy[t], y_perm[pos]>, the logit
//      gradient of the renormalised top-k softmax, dl_j = g_j (dg_j - sum_i
//      g_i dg_i), and for each queue row its token and gate (qtok, qgate);
//   2. grouped GEMMs over the queues: dh_raw = dy W_down with dy's rows
//      gathered by token (the queue rows' output gradient g dy[t] is never
//      stored: the gate comes in the next epilogue), the recompute of
//      gate/up with the SwiGLU backward of dh = g dh_raw, dx_perm; and the
//      weight gradients, which read x and dy by token through qtok and the
//      rest in queue order;
//   3. per token: dx[t] = sum_j dx_perm[pos(t, j)] + sum_j dl_j W_r[id_j];
//   4. router weight gradient dW_r[e] = sum over expert e's queue of dl x:
//      partial sums over each 64-row block of the padded queue (one expert
//      per block), then a second kernel adds an expert's blocks in order.
// All reductions run in a fixed order (deterministic); accumulation is fp32,
// storage bf16.
#include "device_util.h"
#include "moe_internal.h"

namespace moe {

namespace {

// Step 1: each queue row's token and gate, qtok[pos] = a / k and qgate[pos]
// = gates[a] for assignment a at queue position pos; one thread per
// assignment.
__global__ __launch_bounds__(256) void bwd_rows_kernel(const int32_t* __restrict__ assign_pos,
                                                      const float* __restrict__ gates, int k, int64_t n,
                                                      int32_t* __restrict__ qtok, float* __restrict__ qgate) {
    const int64_t a = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (a >= n) return;
    const int pos = assign_pos[a];
    if (pos < 0) return;
    qtok[pos] = static_cast<int32_t>(a / k);
    qgate[pos] = gates[a];
}

// Step 3b, one wave per token: the gate-weighted slot gradients gdg_j =
// g_j <dy[t], y_perm[pos]> from the recompute's partial sums (dg_part
// [T*k][P], P per queue row, summed in a fixed order: lane c adds entries c,
// c + 64, ..., then a butterfly over the lanes), and the logit gradient of
// the renormalised top-k softmax, dsel[t, j] = dl_j = g_j (dg_j - sum_i g_i
// dg_i) = gdg_j - g_j sum_i gdg_i; dlogits (if given) holds dl_j at expert
// id_j and zero elsewhere.
__global__ __launch_bounds__(256) void bwd_dl_kernel(const float* __restrict__ dg_part, int P,
                                                    const int32_t* __restrict__ ids,
                                                    const float* __restrict__ gates,
                                                    const int32_t* __restrict__ assign_pos, int64_t T, int k,
                                                    int E, float* __restrict__ dsel,
                                                    float* __restrict__ dlogits) {
    __shared__ float s_gdg[4][MOE_MAX_TOPK];
    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (t >= T) return;
    // (four slots at a time, their loads in flight together)
    for (int j0 = 0; j0 < k; j0 += 4) {
        int pos[4];
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            pos[u] = j0 + u < k ? assign_pos[t * k + j0 + u] : -1;
            v[u] = 0.f;
        }
        for (int c = lane; c < P; c += 64) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (pos[u] >= 0) v[u] += dg_part[static_cast<int64_t>(pos[u]) * P + c];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v[u] += __shfl_xor(v[u], off, 64);
            if (lane == 0 && j0 + u < k) s_gdg[w][j0 + u] = v[u];
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
    float inner = 0.f;
    for (int j = 0; j < k; ++j) inner += s_gdg[w][j];
    for (int j = lane; j < k; j += 64) dsel[t * k + j] = s_gdg[w][j] - gates[t * k + j] * inner;
    if (dlogits != nullptr) {
        for (int e = lane; e < E; e += 64) {
            float v = 0.f;
            for (int j = 0; j < k; ++j)
                if (ids[t * k + j] == e) v = s_gdg[w][j] - gates[t * k + j] * inner;
            dlogits[t * E + e] = v;
        }
    }
}

// Padded offsets: expert e's queue columns start at poff[e], each expert's
// count rounded up to a multiple of 64 (all zero when offsets is null: no
// tokens).  Also the experts in descending order of padded count, ties by
// lower id: order[rank] = e.  One thread per expert.  And token 0 in the 64
// entries of qtok after the last queue row (a weight gradient's last slice of
// an expert reads up to 63 rows past its end; their values are zeroed, but
// their addresses must be valid).
static_assert(MOE_MAX_EXPERTS == 256, "bwd_poff_kernel runs one 256-thread workgroup, a thread per expert");
__global__ __launch_bounds__(256) void bwd_poff_kernel(const int32_t* __restrict__ offsets, int E,
                                                      int32_t* __restrict__ poff, int32_t* __restrict__ order,
                                                      int32_t* __restrict__ qtok) {
    __shared__ __align__(16) int s_c[MOE_MAX_EXPERTS];
    __shared__ int s_wave[4];
    const int e = threadIdx.x;
    if (offsets != nullptr && e < 64) qtok[offsets[E] + e] = 0;
    const int c = (e < E && offsets != nullptr) ? ((offsets[e + 1] - offsets[e] + 63) / 64) * 64 : 0;
    s_c[e] = c;
    int incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if ((e & 63) >= off) incl += o;
    }
    if ((e & 63) == 63) s_wave[e >> 6] = incl;
    __syncthreads();
    for (int w = 0; w < (e >> 6); ++w) incl += s_wave[w];
    if (e < E) poff[e] = incl - c;
    if (e == E - 1) poff[E] = incl;
    if (e >= E) return;
    // (entries past E hold 0 and never outrank a count >= 0)
    int rank = 0;
    const int4* s4 = reinterpret_cast<const int4*>(s_c);
#pragma unroll 8
    for (int o4 = 0; o4 < MOE_MAX_EXPERTS / 4; ++o4) {
        const int4 v = s4[o4];
        const int o = o4 * 4;
        rank += (v.x > c || (v.x == c && o < e)) ? 1 : 0;
        rank += (v.y > c || (v.y == c && o + 1 < e)) ? 1 : 0;
        rank += (v.z > c || (v.z == c && o + 2 < e)) ? 1 : 0;
        rank += (v.w > c || (v.w == c && o + 3 < e)) ? 1 : 0;
    }
    order[rank] = e;
}

// The router gradient's partial sums over the queues.  The grid walks each
// expert's queue in 64-row blocks of the padded queue (expert e's rows start
// at padded row poff[e], a multiple of 64, so a block belongs to one expert;
// padded row q is queue row pos = offsets[e] + q - poff[e] while pos <
// offsets[e+1], else padding) and kGatherXCols columns at a time.  Block b =
// q / 64 yields wr_part[b, c] = sum over its rows of dsel[a] x[a / k, c] (a =
// sorted_assign[pos]; padding adds nothing), in a fixed order: wave w adds
// rows 16w .. 16w + 15 in turn (each lane 8 columns, its 16 row loads in
// flight first), then (s0 + s1) + (s2 + s3) over the waves.
constexpr int kGatherXCols = 512;
__global__ __launch_bounds__(256) void bwd_router_partials_kernel(const bf16_t* __restrict__ x, int d,
                                                                 const int32_t* __restrict__ offsets,
                                                                 const int32_t* __restrict__ poff, int E,
                                                                 const int32_t* __restrict__ sorted_assign,
                                                                 int k, const float* __restrict__ dsel,
                                                                 float* __restrict__ wr_part) {
    __shared__ int64_t s_row[64];
    __shared__ float s_dsel[64];
    __shared__ float s_part[4][kGatherXCols];
    __shared__ int s_poff[MOE_MAX_EXPERTS + 1];
    const int q0 = blockIdx.x * 64;
    const int c0 = blockIdx.y * kGatherXCols;
    if (q0 >= poff[E]) return;
    // the padded offsets in LDS with one load per thread, so that the search
    // below costs no global round trips
    for (int i = threadIdx.x; i <= E; i += 256) s_poff[i] = poff[i];
    __syncthreads();
    if (threadIdx.x < 64) {
        const int q = q0 + threadIdx.x;
        int lo = 0, hi = E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_poff[mid] <= q) lo = mid; else hi = mid;
        }
        const int pos = offsets[lo] + (q - s_poff[lo]);
        int64_t row = -1;
        float ds = 0.f;
        if (pos < offsets[lo + 1]) {
            const int a = sorted_assign[pos];
            row = a / k;
            ds = dsel[a];
        }
        s_row[threadIdx.x] = row;
        s_dsel[threadIdx.x] = ds;
    }
    __syncthreads();
    const int w = threadIdx.x >> 6;
    const int cl = (threadIdx.x & 63) * 8;  // the lane's 8 columns within the strip
    const int c = c0 + cl;
    float part[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < d) {
        // branch-free: a padding row loads x row 0 and keeps zeros
        uint4 v[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = s_row[w * 16 + r];
            const uint4 t = *reinterpret_cast<const uint4*>(x + (row >= 0 ? row : 0) * d + c);
            v[r] = row >= 0 ? t : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float ds = s_dsel[w * 16 + r];
            const uint32_t u[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                part[2 * h] = fmaf(ds, __uint_as_float(u[h] << 16), part[2 * h]);
                part[2 * h + 1] = fmaf(ds, __uint_as_float(u[h] & 0xffff0000u), part[2 * h + 1]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s_part[w][cl + i] = part[i];
    __syncthreads();
    for (int i = threadIdx.x; i < kGatherXCols; i += 256) {
        if (c0 + i < d)
            wr_part[static_cast<int64_t>(q0 / 64) * d + c0 + i] =
                (s_part[0][i] + s_part[1][i]) + (s_part[2][i] + s_part[3][i]);
    }
}

// Step 3: dx[t] = sum_j dx_perm[pos(t, j)] (+ sum_j dl_j W_r[id_j]), fp32 in
// ascending j, one rounding.  KM > 0: k <= KM, the token's positions (ids,
// logit gradients) read once into LDS and a chunk's k row loads issued
// together; KM = 0: any k, one row at a time.  Same sums either way.
template <int KM>
__global__ __launch_bounds__(256) void bwd_dx_kernel(const uint4* __restrict__ dx_perm,
                                                    const int32_t* __restrict__ assign_pos,
                                                    const int32_t* __restrict__ ids,
                                                    const float* __restrict__ dsel,
                                                    const uint4* __restrict__ w_router, int k, int E,
                                                    int chunks, uint4* __restrict__ dx) {
    const int64_t t = blockIdx.x;
    if constexpr (KM > 0) {
        __shared__ int s_pos[KM];
        __shared__ int s_e[KM];
        __shared__ float s_dl[KM];
        if (threadIdx.x < KM) {
            const int j = threadIdx.x;
            s_pos[j] = j < k ? assign_pos[t * k + j] : -1;
            const int e = j < k && w_router != nullptr ? ids[t * k + j] : -1;
            s_e[j] = static_cast<unsigned>(e) < static_cast<unsigned>(E) ? e : -1;
            s_dl[j] = j < k && w_router != nullptr ? dsel[t * k + j] : 0.f;
        }
        __syncthreads();
        int pos[KM], ex[KM];
        float dl[KM];
#pragma unroll
        for (int j = 0; j < KM; ++j) {
            pos[j] = s_pos[j];
            ex[j] = s_e[j];
            dl[j] = s_dl[j];
        }
        for (int c = threadIdx.x; c < chunks; c += 256) {
            uint4 v[KM];
#pragma unroll
            for (int j = 0; j < KM; ++j)
                v[j] = pos[j] >= 0 ? load_nt(dx_perm + static_cast<int64_t>(pos[j]) * chunks + c)
                                   : make_uint4(0u, 0u, 0u, 0u);
            uint4 wr[KM];
            if (w_router != nullptr) {
#pragma unroll
                for (int j = 0; j < KM; ++j)
                    wr[j] = ex[j] >= 0 ? w_router[static_cast<int64_t>(ex[j]) * chunks + c] : make_uint4(0u, 0u, 0u, 0u);
            }
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
            for (int j = 0; j < KM; ++j) {
                if (pos[j] < 0) continue;
                const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += lo_bf16(w[i]);
                    acc[2 * i + 1] += hi_bf16(w[i]);
                }
            }
            if (w_router != nullptr) {
#pragma unroll
                for (int j = 0; j < KM; ++j) {
                    if (ex[j] < 0) continue;
                    const uint32_t w[4] = {wr[j].x, wr[j].y, wr[j].z, wr[j].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] = fmaf(dl[j], lo_bf16(w[i]), acc[2 * i]);
                        acc[2 * i + 1] = fmaf(dl[j], hi_bf16(w[i]), acc[2 * i + 1]);
                    }
                }
            }
            dx[t * chunks + c] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                            pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
        }
        return;
    }
    for (int c = threadIdx.x; c < chunks; c += 256) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
        for (int j = 0; j < k; ++j) {
            const int pos = assign_pos[t * k + j];
            if (pos < 0) continue;
            const uint4 v = load_nt(dx_perm + static_cast<int64_t>(pos) * chunks + c);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += lo_bf16(w[i]);
                acc[2 * i + 1] += hi_bf16(w[i]);
            }
        }
        if (w_router != nullptr) {
            for (int j = 0; j < k; ++j) {
                const int e = ids[t * k + j];
                if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) continue;
                const float dl = dsel[t * k + j];
                const uint4 v = w_router[static_cast<int64_t>(e) * chunks + c];
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] = fmaf(dl, lo_bf16(w[i]), acc[2 * i]);
                    acc[2 * i + 1] = fmaf(dl, hi_bf16(w[i]), acc[2 * i + 1]);
                }
            }
        }
        dx[t * chunks + c] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                        pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
}

// Step 4: dW_r[e, c] = sum of the partial sums of expert e's 64-column
// blocks [poff[e] / 64, poff[e+1] / 64), ascending; grid (E, d / 256), one
// column per thread.
__global__ __launch_bounds__(256) void bwd_dwr_kernel(const float* __restrict__ wr_part,
                                                     const int32_t* __restrict__ poff, int d,
                                                     bf16_t* __restrict__ dw_router) {
    const int e = blockIdx.x;
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= d) return;
    float acc = 0.f;
    const int b1 = poff[e + 1] / 64;
    // (unrolled so that the loads of 8 blocks are in flight together; the
    // sum stays in block order)
#pragma unroll 8
    for (int b = poff[e] / 64; b < b1; ++b) acc += wr_part[static_cast<int64_t>(b) * d + c];
    dw_router[static_cast<int64_t>(e) * d + c] = __builtin_bit_cast(bf16_t, static_cast<__bf16>(acc));
}

// Weight transpose for the backward GEMMs, per expert (gridDim.z):
// dst[e][c][col0 + i] = src[e][i][c] for i < R, c < Cc (src rows of Cc,
// dst rows of ld_dst).  Tiles of 64 x 64 through LDS.
__global__ __launch_bounds__(256) void weight_transpose_kernel(const bf16_t* __restrict__ src, int R,
                                                              int Cc, bf16_t* __restrict__ dst,
                                                              int64_t ld_dst, int col0) {
    __shared__ bf16_t tile[64][64 + 2];
    const int64_t e = blockIdx.z;
    const int i0 = blockIdx.x * 64;
    const int c0 = blockIdx.y * 64;
    const bf16_t* s = src + e * R * Cc;
    bf16_t* dd = dst + e * Cc * ld_dst;
    {
        const int i = threadIdx.x >> 2;
        const int cc = (threadIdx.x & 3) * 16;
#pragma unroll
        for (int u = 0; u < 16; u += 8) {
            const int c = c0 + cc + u;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (i0 + i < R && c < Cc) v = *reinterpret_cast<const uint4*>(s + static_cast<int64_t>(i0 + i) * Cc + c);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                tile[i][cc + u + 2 * h] = static_cast<bf16_t>(w[h] & 0xffffu);
                tile[i][cc + u + 2 * h + 1] = static_cast<bf16_t>(w[h] >> 16);
            }
        }
    }
    __syncthreads();
    {
        const int c = threadIdx.x >> 2;
        const int ii = (threadIdx.x & 3) * 16;
        if (c0 + c < Cc) {
#pragma unroll
            for (int u = 0; u < 16; u += 8) {
                if (i0 + ii + u >= R) continue;
                uint32_t w[4];
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    w[h] = static_cast<uint32_t>(tile[ii + u + 2 * h][c]) |
                           (static_cast<uint32_t>(tile[ii + u + 2 * h + 1][c]) << 16);
                *reinterpret_cast<uint4*>(dd + static_cast<int64_t>(c0 + c) * ld_dst + col0 + i0 + ii + u) =
                    make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }
}

}  // namespace

hipError_t launch_backward_weights(const moe_problem_t& p, const void* w_gate, const void* w_up,
                                   const void* w_down, void* w_down_t, void* w_gu_t, hipStream_t s) {
    // W_down [E, d, f] -> W_down_t [E, f, d]
    weight_transpose_kernel<<<dim3(ceil_div(p.d, 64), ceil_div(p.f, 64), p.E), 256, 0, s>>>(
        static_cast<const bf16_t*>(w_down), p.d, p.f, static_cast<bf16_t*>(w_down_t), p.d, 0);
    // W_gate, W_up [E, f, d] -> W_gu_t [E, d, 2f] (gate columns, then up columns)
    const dim3 g(ceil_div(p.f, 64), ceil_div(p.d, 64), p.E);
    weight_transpose_kernel<<<g, 256, 0, s>>>(static_cast<const bf16_t*>(w_gate), p.f, p.d,
                                              static_cast<bf16_t*>(w_gu_t), 2 * int64_t{p.f}, 0);
    weight_transpose_kernel<<<g, 256, 0, s>>>(static_cast<const bf16_t*>(w_up), p.f, p.d,
                                              static_cast<bf16_t*>(w_gu_t), 2 * int64_t{p.f}, p.f);
    return hipGetLastError();
}

hipError_t launch_backward_rows(const moe_problem_t& p, const int32_t* assign_pos, const float* gates,
                                int32_t* qtok, float* qgate, hipStream_t s) {
    const int64_t n = p.T * p.k;
    bwd_rows_kernel<<<static_cast<unsigned>(ceil_div(n, 256)), 256, 0, s>>>(assign_pos, gates, p.k, n, qtok,
                                                                            qgate);
    return hipGetLastError();
}

hipError_t launch_backward_dl(const moe_problem_t& p, const float* dg_part, const int32_t* ids,
                              const float* gates, const int32_t* assign_pos, float* dsel, float* dlogits,
                              hipStream_t s) {
    bwd_dl_kernel<<<static_cast<unsigned>(ceil_div(p.T, 4)), 256, 0, s>>>(
        dg_part, bwd_dg_parts(p), ids, gates, assign_pos, p.T, p.k, p.E, dsel, dlogits);
    return hipGetLastError();
}

hipError_t launch_backward_poff(const moe_problem_t& p, const int32_t* offsets, int32_t* poff,
                                int32_t* order, int32_t* qtok, hipStream_t s) {
    bwd_poff_kernel<<<1, 256, 0, s>>>(offsets, p.E, poff, order, qtok);
    return hipGetLastError();
}

hipError_t launch_backward_router_partials(const moe_problem_t& p, const void* x, const int32_t* offsets,
                                           const int32_t* poff, const int32_t* sorted_assign, int64_t kpad,
                                           const float* dsel, float* wr_part, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(kpad / 64), static_cast<unsigned>(ceil_div(p.d, kGatherXCols)));
    bwd_router_partials_kernel<<<grid, 256, 0, s>>>(static_cast<const bf16_t*>(x), p.d, offsets, poff, p.E,
                                                    sorted_assign, p.k, dsel, wr_part);
    return hipGetLastError();
}

hipError_t launch_backward_dx(const moe_problem_t& p, const void* dx_perm, const int32_t* assign_pos,
                              const int32_t* ids, const float* dsel, const void* w_router, void* dx,
                              hipStream_t s) {
    const unsigned grid = static_cast<unsigned>(p.T);
    const uint4* src = static_cast<const uint4*>(dx_perm);
    const uint4* wr = static_cast<const uint4*>(w_router);
    uint4* out = static_cast<uint4*>(dx);
    if (p.k <= 2)
        bwd_dx_kernel<2><<<grid, 256, 0, s>>>(src, assign_pos, ids, dsel, wr, p.k, p.E, p.d / 8, out);
    else if (p.k <= 4)
        bwd_dx_kernel<4><<<grid, 256, 0, s>>>(src, assign_pos, ids, dsel, wr, p.k, p.E, p.d / 8, out);
    else if (p.k <= 8)
        bwd_dx_kernel<8><<<grid, 256, 0, s>>>(src, assign_pos, ids, dsel, wr, p.k, p.E, p.d / 8, out);
    else
        bwd_dx_kernel<0><<<grid, 256, 0, s>>>(src, assign_pos, ids, dsel, wr, p.k, p.E, p.d / 8, out);
    return hipGetLastError();
}

hipError_t launch_backward_dwr(const moe_problem_t& p, const float* wr_part, const int32_t* poff,
                               void* dw_router, hipStream_t s) {
    bwd_dwr_kernel<<<dim3(p.E, ceil_div(p.d, 256)), 256, 0, s>>>(wr_part, poff, p.d,
                                                                static_cast<bf16_t*>(dw_router));
    return hipGetLastError();
}

}  // namespace moe
