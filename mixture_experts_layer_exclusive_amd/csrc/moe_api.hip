// C-ABI entry points: argument validation (pure host code, before any HIP
// call), workspace carving and kernel launches on the caller's stream.
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "moe.h"
#include "moe_internal.h"

using namespace moe;

// Scratch of moe_dispatch_no_alloc: the dispatch's per-block expert count
// table (dispatch_blocks(T*k) x E int32), in a device array of its own so
// that the call needs no workspace argument.  Each GPU the library runs on
// holds one copy, at its own address, until the process ends.  Host code
// never passes `scratch` itself to a kernel (on the host the name stands
// for a host-side shadow, not a device address): it uses the address
// hipGetSymbolAddress returns for the device (scratch_address below).
static __device__ __align__(256) int32_t scratch[MOE_NO_ALLOC_SCRATCH_BYTES / 4];

namespace {

constexpr int32_t kAbiVersion = 4;
constexpr size_t kAlign = 256;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

size_t elem_bytes(const moe_problem_t& p) { return p.dtype == MOE_DTYPE_F32 ? 4 : 2; }

// Checks the problem statement itself.
moe_status_t check_problem(const moe_problem_t* p) {
    if (p == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (p->T < 0 || p->d < 1 || p->E < 1 || p->k < 1 || p->f < 1) return MOE_ERR_INVALID_ARGUMENT;
    if (p->k > p->E) return MOE_ERR_INVALID_ARGUMENT;
    if (p->dtype != MOE_DTYPE_F32 && p->dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARGUMENT;
    if (p->E > MOE_MAX_EXPERTS || p->k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
    if (p->T > INT32_MAX / p->k) return MOE_ERR_UNSUPPORTED;
    // a launch counts its work-items in 32 bits: the per-token kernels run
    // up to 256 lanes per token, the expert FFN 256 per workgroup
    if (p->T > kMaxLaunchItems / 256) return MOE_ERR_UNSUPPORTED;
    if (p->dtype == MOE_DTYPE_BF16 && (p->d % 64 != 0 || p->f % 64 != 0)) return MOE_ERR_UNSUPPORTED;
    // the bf16 GEMMs address one expert's weight matrix with 32-bit byte offsets
    if (p->dtype == MOE_DTYPE_BF16 && static_cast<int64_t>(p->d) * p->f > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    if (expert_ffn_grid_bound(*p) > kMaxLaunchItems / 256) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// A required device pointer: present and 16-byte aligned.
moe_status_t need(const void* ptr) {
    if (ptr == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    return aligned16(ptr) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

// An optional device pointer: NULL, or 16-byte aligned.
moe_status_t optional(const void* ptr) {
    return (ptr == nullptr || aligned16(ptr)) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

#define MOE_TRY(expr)                              \
    do {                                           \
        const moe_status_t st_ = (expr);           \
        if (st_ != MOE_OK) return st_;             \
    } while (0)

#define MOE_LAUNCH(expr)                           \
    do {                                           \
        if ((expr) != hipSuccess) return MOE_ERR_HIP; \
    } while (0)

// Sequential carving of a workspace into 256-byte aligned pieces.
struct Carver {
    uintptr_t base;
    size_t used = 0;
    explicit Carver(void* b) : base(reinterpret_cast<uintptr_t>(b)) {}
    template <typename T>
    T* take(size_t bytes) {
        T* r = reinterpret_cast<T*>(base + used);
        used = align_up(used + bytes, kAlign);
        return r;
    }
};

size_t dispatch_ws(const moe_problem_t& p) {
    const int64_t n = p.T * p.k;
    return align_up(static_cast<size_t>(dispatch_blocks(n)) * p.E * 4, kAlign);
}

size_t ffn_ws(const moe_problem_t& p) { return ffn_h_bytes(p) + ffn_split_bytes(p); }

// Backward workspace: dsel [T*k] fp32; each queue row's token qtok [T*k +
// pad] and gate qgate [T*k] fp32; the slot gradients' partial sums [T*k,
// bwd_dg_parts] fp32; dx_perm [T*k, d]; dh_raw [T*k, f]; g h [T*k + pad, f];
// du|dv [T*k + pad, 2f]; padded offsets [E+1] and the expert order [E]; the
// router-gradient partial sums [kpad / 64, d] fp32; the split-K partial
// tiles of the dx_perm GEMM.  g h and du|dv are the weight
// gradients' queue-order operands (pad = kWgradPadRows rows after the last
// queue row); x and dy are read by token through qtok, never copied into
// queue order.
size_t backward_ws(const moe_problem_t& p) {
    const size_t n = static_cast<size_t>(p.T) * p.k;
    const size_t np = n + static_cast<size_t>(kWgradPadRows);
    const size_t kp = static_cast<size_t>(backward_kpad(p));
    size_t b = align_up(n * 4, kAlign);              // dsel
    b += align_up(np * 4, kAlign);                   // qtok
    b += align_up(n * 4, kAlign);                    // qgate
    b += align_up(n * bwd_dg_parts(p) * 4, kAlign);  // slot-gradient partial sums
    b += align_up(n * p.d * 2, kAlign);              // dx_perm
    b += align_up(n * p.f * 2, kAlign);              // dh_raw
    b += align_up(np * p.f * 2, kAlign);             // g h
    b += align_up(np * 2 * p.f * 2, kAlign);         // du|dv
    b += align_up(static_cast<size_t>(p.E + 1) * 4, kAlign);
    b += align_up(static_cast<size_t>(p.E) * 4, kAlign);           // expert order
    b += align_up(static_cast<size_t>(kp / 64) * p.d * 4, kAlign);
    b += align_up(bwd_split_bytes(p), kAlign);
    return b;
}

// Limits of the bf16 backward (beyond check_problem): the GEMMs address
// [E, d, 2f] weight rows with 32-bit byte offsets, and the recompute's gather
// of x takes 32-bit offsets too (T * d below 2^31).
moe_status_t check_backward(const moe_problem_t* p) {
    if (p->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(p->d) * p->f >= (int64_t{1} << 30)) return MOE_ERR_UNSUPPORTED;
    if (p->T * static_cast<int64_t>(p->d) >= (int64_t{1} << 31)) return MOE_ERR_UNSUPPORTED;
    if (backward_kpad(*p) > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

// fp8 expert FFN workspace: x codes [T, d] and exponents [T], h codes
// [T*k, f] and their E8M0 scales (one byte per 32 columns), split-K partial
// tiles.
size_t ffn_fp8_ws(const moe_problem_t& p) {
    const size_t n = static_cast<size_t>(p.T) * p.k;
    return align_up(static_cast<size_t>(p.T) * p.d, kAlign) + align_up(static_cast<size_t>(p.T) * 4, kAlign) +
           align_up(n * p.f, kAlign) + align_up(n * (p.f / 32), kAlign) + align_up(fp8_split_bytes(p), kAlign);
}

// Limits of the fp8 path (beyond check_problem): bf16 weights and
// activations, d and f multiples of 128 (one 128-byte slice of codes), and
// 32-bit byte offsets into the x codes.
moe_status_t check_fp8(const moe_problem_t* p) {
    if (p->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->d % 128 != 0 || p->f % 128 != 0) return MOE_ERR_UNSUPPORTED;
    if (p->T * static_cast<int64_t>(p->d) > UINT32_MAX) return MOE_ERR_UNSUPPORTED;
    // the weight quantisation takes every weight row as one row of a launch
    if (static_cast<int64_t>(p->E) * std::max(p->d, p->f) > kMaxLaunchItems / 256) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

size_t forward_ws(const moe_problem_t& p) {
    const size_t n = static_cast<size_t>(p.T) * p.k;
    size_t b = 0;
    b += align_up(static_cast<size_t>(p.T) * p.E * 4, kAlign);  // logits
    b += align_up(n * 4, kAlign) * 4;                           // ids, gates, sorted_assign, assign_pos
    b += align_up(static_cast<size_t>(p.E) * 4, kAlign);       // counts
    b += align_up(static_cast<size_t>(p.E + 1) * 4, kAlign);   // offsets
    b += dispatch_ws(p);                                        // block counts
    b += ffn_ws(p);                                             // h, split-K partials
    b += align_up(n * p.d * elem_bytes(p), kAlign);             // y_perm
    return b;
}

void clear_hip_error() { (void)hipGetLastError(); }

// Device address of `scratch` on the device of stream s: looked up once per
// device, with that device current (the caller's current device is restored),
// then kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

hipError_t scratch_address(hipStream_t s, void** out) {
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(s, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* addr = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (addr == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        addr = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (addr == nullptr) {
            int cur = 0;
            if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (cur != dev) {
                const hipError_t e2 = hipSetDevice(cur);
                if (e == hipSuccess) e = e2;
            }
            if (e != hipSuccess) return e;
            if (addr == nullptr) return hipErrorInvalidSymbol;
            g_scratch_addr[dev].store(addr, std::memory_order_release);
        }
    }
    *out = addr;
    return hipSuccess;
}

}  // namespace

extern "C" {

const char* moe_status_string(int32_t status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

int32_t moe_abi_version(void) { return kAbiVersion; }

moe_status_t moe_workspace_size(const moe_problem_t* p, int32_t op, size_t* bytes) {
    if (bytes == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(check_problem(p));
    switch (op) {
        case MOE_OP_DISPATCH: *bytes = dispatch_ws(*p); break;
        case MOE_OP_EXPERT_FFN: *bytes = ffn_ws(*p); break;
        case MOE_OP_FORWARD: *bytes = forward_ws(*p); break;
        case MOE_OP_BACKWARD:
            MOE_TRY(check_backward(p));
            *bytes = backward_ws(*p);
            break;
        case MOE_OP_EXPERT_FFN_FP8:
            MOE_TRY(check_fp8(p));
            *bytes = ffn_fp8_ws(*p);
            break;
        default: return MOE_ERR_INVALID_ARGUMENT;
    }
    return MOE_OK;
}

moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_router,
                       const float* logits_in, float* logits_out, int32_t* topk_ids,
                       float* topk_gates, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return MOE_OK;
    if (logits_in != nullptr) {
        MOE_TRY(need(logits_in));
    } else {
        // the router GEMM writes its logits to logits_out, then top-k reads them
        MOE_TRY(need(x));
        MOE_TRY(need(w_router));
        MOE_TRY(need(logits_out));
    }
    MOE_TRY(need(topk_ids));
    MOE_TRY(need(topk_gates));
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    const float* l = logits_in;
    if (l == nullptr) {
        MOE_LAUNCH(launch_router_logits(*p, x, w_router, logits_out, s));
        l = logits_out;
    }
    MOE_LAUNCH(launch_route_topk(*p, l, topk_ids, topk_gates, s));
    return MOE_OK;
}

moe_status_t moe_dispatch(const moe_problem_t* p, const int32_t* topk_ids, const void* x,
                          int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                          int32_t* assign_pos, void* x_perm, void* ws, size_t ws_bytes,
                          void* stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return MOE_OK;
    MOE_TRY(need(topk_ids));
    MOE_TRY(need(counts));
    MOE_TRY(need(offsets));
    MOE_TRY(need(sorted_assign));
    MOE_TRY(need(assign_pos));
    MOE_TRY(optional(x_perm));
    if (x_perm != nullptr) MOE_TRY(need(x));
    MOE_TRY(need(ws));
    if (ws_bytes < dispatch_ws(*p)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    MOE_LAUNCH(launch_dispatch(*p, topk_ids, x, counts, offsets, sorted_assign, assign_pos,
                               static_cast<int32_t*>(ws), x_perm, s));
    return MOE_OK;
}

moe_status_t moe_dispatch_no_alloc(const moe_problem_t* p, const int32_t* topk_ids, const void* x,
                                   int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                                   int32_t* assign_pos, void* x_perm, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return MOE_OK;
    MOE_TRY(need(topk_ids));
    MOE_TRY(need(counts));
    MOE_TRY(need(offsets));
    MOE_TRY(need(sorted_assign));
    MOE_TRY(need(assign_pos));
    MOE_TRY(optional(x_perm));
    if (x_perm != nullptr) MOE_TRY(need(x));
    // the count table must fit the static scratch
    if (dispatch_ws(*p) > MOE_NO_ALLOC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    void* table = nullptr;
    if (scratch_address(s, &table) != hipSuccess) return MOE_ERR_HIP;
    // (the histogram writes every entry of the table that the scatter, or
    // the one-pass scatter and gather, reads, so nothing in it has to start
    // at zero)
    MOE_LAUNCH(launch_dispatch(*p, topk_ids, x, counts, offsets, sorted_assign, assign_pos,
                               static_cast<int32_t*>(table), x_perm, s));
    return MOE_OK;
}

moe_status_t moe_expert_ffn(const moe_problem_t* p, const void* x_perm, const void* x,
                            const int32_t* sorted_assign, const int32_t* offsets,
                            const void* w_gate, const void* w_up, const void* w_down,
                            void* y_perm, void* ws, size_t ws_bytes, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return MOE_OK;
    if (x_perm != nullptr) {
        MOE_TRY(need(x_perm));
    } else {
        MOE_TRY(need(x));
        MOE_TRY(need(sorted_assign));
    }
    MOE_TRY(need(offsets));
    MOE_TRY(need(w_gate));
    MOE_TRY(need(w_up));
    MOE_TRY(need(w_down));
    MOE_TRY(need(y_perm));
    MOE_TRY(need(ws));
    if (ws_bytes < ffn_ws(*p)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    MOE_LAUNCH(launch_expert_ffn(*p, x_perm, x, sorted_assign, offsets, w_gate, w_up, w_down, ws,
                                 y_perm, s));
    return MOE_OK;
}

moe_status_t moe_combine(const moe_problem_t* p, const void* y_perm, const int32_t* assign_pos,
                         const float* topk_gates, void* y, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return MOE_OK;
    MOE_TRY(need(y_perm));
    MOE_TRY(need(assign_pos));
    MOE_TRY(need(topk_gates));
    MOE_TRY(need(y));
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    MOE_LAUNCH(launch_combine(*p, y_perm, assign_pos, topk_gates, y, s));
    return MOE_OK;
}

moe_status_t moe_forward(const moe_problem_t* p, const void* x, const void* w_router,
                         const float* logits_in, const void* w_gate, const void* w_up,
                         const void* w_down, void* y, const moe_forward_outputs_t* out, void* ws,
                         size_t ws_bytes, void* stream) {
    MOE_TRY(check_problem(p));
    if (p->T == 0) return MOE_OK;
    MOE_TRY(need(x));
    if (logits_in != nullptr) MOE_TRY(need(logits_in));
    else MOE_TRY(need(w_router));
    MOE_TRY(need(w_gate));
    MOE_TRY(need(w_up));
    MOE_TRY(need(w_down));
    MOE_TRY(need(y));
    moe_forward_outputs_t o = {};
    if (out != nullptr) {
        o = *out;
        MOE_TRY(optional(o.logits));
        MOE_TRY(optional(o.topk_ids));
        MOE_TRY(optional(o.topk_gates));
        MOE_TRY(optional(o.counts));
        MOE_TRY(optional(o.offsets));
        MOE_TRY(optional(o.sorted_assign));
        MOE_TRY(optional(o.assign_pos));
        MOE_TRY(optional(o.y_perm));
    }
    MOE_TRY(need(ws));
    if (ws_bytes < forward_ws(*p)) return MOE_ERR_WORKSPACE_TOO_SMALL;

    const size_t n = static_cast<size_t>(p->T) * p->k;
    Carver c(ws);
    float* logits = c.take<float>(static_cast<size_t>(p->T) * p->E * 4);
    int32_t* ids = c.take<int32_t>(n * 4);
    float* gates = c.take<float>(n * 4);
    int32_t* sa = c.take<int32_t>(n * 4);
    int32_t* ap = c.take<int32_t>(n * 4);
    int32_t* counts = c.take<int32_t>(static_cast<size_t>(p->E) * 4);
    int32_t* offsets = c.take<int32_t>(static_cast<size_t>(p->E + 1) * 4);
    int32_t* bc = c.take<int32_t>(dispatch_ws(*p));
    void* h = c.take<char>(ffn_ws(*p));
    void* y_perm = c.take<char>(n * p->d * elem_bytes(*p));
    if (o.logits) logits = o.logits;
    if (o.topk_ids) ids = o.topk_ids;
    if (o.topk_gates) gates = o.topk_gates;
    if (o.sorted_assign) sa = o.sorted_assign;
    if (o.assign_pos) ap = o.assign_pos;
    if (o.counts) counts = o.counts;
    if (o.offsets) offsets = o.offsets;
    if (o.y_perm) y_perm = o.y_perm;

    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    const float* l = logits_in;
    if (l == nullptr) {
        MOE_LAUNCH(launch_router_logits(*p, x, w_router, logits, s));
        l = logits;
    }
    MOE_LAUNCH(launch_route_topk(*p, l, ids, gates, s));
    MOE_LAUNCH(launch_dispatch_queues(*p, ids, counts, offsets, sa, ap, bc, s));
    MOE_LAUNCH(launch_expert_ffn(*p, nullptr, x, sa, offsets, w_gate, w_up, w_down, h, y_perm, s));
    MOE_LAUNCH(launch_combine(*p, y_perm, ap, gates, y, s));
    return MOE_OK;
}

moe_status_t moe_backward_weights(const moe_problem_t* p, const void* w_gate, const void* w_up,
                                  const void* w_down, void* w_down_t, void* w_gu_t, void* stream) {
    MOE_TRY(check_problem(p));
    MOE_TRY(check_backward(p));
    MOE_TRY(need(w_gate));
    MOE_TRY(need(w_up));
    MOE_TRY(need(w_down));
    MOE_TRY(need(w_down_t));
    MOE_TRY(need(w_gu_t));
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    MOE_LAUNCH(launch_backward_weights(*p, w_gate, w_up, w_down, w_down_t, w_gu_t, s));
    return MOE_OK;
}

moe_status_t moe_backward(const moe_problem_t* p, const void* x, const void* w_router,
                          const void* w_gate, const void* w_up, const void* w_down_t,
                          const void* w_gu_t, const moe_forward_state_t* fw, const void* dy,
                          const moe_backward_outputs_t* out, void* ws, size_t ws_bytes,
                          void* stream) {
    MOE_TRY(check_problem(p));
    MOE_TRY(check_backward(p));
    if (fw == nullptr || out == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(need(w_gate));
    MOE_TRY(need(w_up));
    MOE_TRY(need(w_down_t));
    MOE_TRY(need(w_gu_t));
    MOE_TRY(need(out->dw_gate));
    MOE_TRY(need(out->dw_up));
    MOE_TRY(need(out->dw_down));
    MOE_TRY(optional(out->dlogits));
    if (w_router != nullptr) {
        MOE_TRY(need(w_router));
        MOE_TRY(need(out->dw_router));
    } else if (out->dw_router != nullptr) {
        return MOE_ERR_INVALID_ARGUMENT;
    }
    if (p->T > 0) {
        MOE_TRY(need(x));
        MOE_TRY(need(dy));
        MOE_TRY(need(out->dx));
        MOE_TRY(need(fw->offsets));
        MOE_TRY(need(fw->topk_ids));
        MOE_TRY(need(fw->topk_gates));
        MOE_TRY(need(fw->sorted_assign));
        MOE_TRY(need(fw->assign_pos));
    }
    MOE_TRY(need(ws));
    if (ws_bytes < backward_ws(*p)) return MOE_ERR_WORKSPACE_TOO_SMALL;

    const size_t n = static_cast<size_t>(p->T) * p->k;
    const size_t np = n + static_cast<size_t>(kWgradPadRows);
    const int64_t kp = backward_kpad(*p);
    Carver c(ws);
    float* dsel = c.take<float>(n * 4);
    int32_t* qtok = c.take<int32_t>(np * 4);
    float* qgate = c.take<float>(n * 4);
    float* dg_part = c.take<float>(n * bwd_dg_parts(*p) * 4);
    void* dx_perm = c.take<char>(n * p->d * 2);
    void* dh = c.take<char>(n * p->f * 2);
    void* hg = c.take<char>(np * p->f * 2);
    void* duv = c.take<char>(np * 2 * p->f * 2);
    int32_t* poff = c.take<int32_t>(static_cast<size_t>(p->E + 1) * 4);
    int32_t* order = c.take<int32_t>(static_cast<size_t>(p->E) * 4);
    float* wr_part = c.take<float>(static_cast<size_t>(kp / 64) * p->d * 4);
    float* split = bwd_split_bytes(*p) > 0 ? c.take<float>(bwd_split_bytes(*p)) : nullptr;

    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    // (with no tokens fw is not read: every queue is empty)
    MOE_LAUNCH(launch_backward_poff(*p, p->T > 0 ? fw->offsets : nullptr, poff, order, qtok, s));
    if (p->T > 0) {
        MOE_LAUNCH(launch_backward_rows(*p, fw->assign_pos, fw->topk_gates, qtok, qgate, s));
        MOE_LAUNCH(launch_backward_dh(*p, dy, fw->sorted_assign, fw->offsets, w_down_t, dh, s));
        MOE_LAUNCH(launch_backward_recompute(*p, x, fw->sorted_assign, fw->offsets, w_gate, w_up, dh, qgate,
                                             duv, hg, dg_part, s));
        MOE_LAUNCH(launch_backward_dl(*p, dg_part, fw->topk_ids, fw->topk_gates, fw->assign_pos, dsel,
                                      out->dlogits, s));
        MOE_LAUNCH(launch_backward_dxperm(*p, duv, fw->offsets, w_gu_t, dx_perm, split, s));
        MOE_LAUNCH(launch_backward_dx(*p, dx_perm, fw->assign_pos, fw->topk_ids, dsel, w_router, out->dx,
                                      s));
        // with a router, its gradient's partial sums over 64-row blocks of
        // each queue
        if (w_router != nullptr)
            MOE_LAUNCH(launch_backward_router_partials(*p, x, fw->offsets, poff, fw->sorted_assign, kp, dsel,
                                                       wr_part, s));
    }
    // weight gradients: dW_down from dy (by token) and g h, dW_gate and dW_up
    // from du, dv and x (by token); an expert with no rows gets zeros (with
    // no tokens every count, from poff, is zero, and qtok is not read)
    // (du and dv are columns 0 .. f and f .. 2f of du|dv)
    const int32_t* qoff = p->T > 0 ? fw->offsets : poff;
    MOE_LAUNCH(launch_backward_wgrad(*p, dy, p->d, 0, p->d, hg, p->f, qoff, order, qtok, false, out->dw_down,
                                     s));
    MOE_LAUNCH(launch_backward_wgrad(*p, duv, 2 * p->f, 0, p->f, x, p->d, qoff, order, qtok, true, out->dw_gate,
                                     s));
    MOE_LAUNCH(launch_backward_wgrad(*p, duv, 2 * p->f, p->f, p->f, x, p->d, qoff, order, qtok, true, out->dw_up,
                                     s));
    if (w_router != nullptr)
        MOE_LAUNCH(launch_backward_dwr(*p, wr_part, poff, out->dw_router, s));
    return MOE_OK;
}

moe_status_t moe_quantize_rows_fp8(const void* src, int64_t rows, int32_t cols, void* codes, int32_t* exps,
                                   void* stream) {
    if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARGUMENT;
    // (one 256-lane workgroup per row at most: 32-bit work-item count)
    if (rows > kMaxLaunchItems / 256 || cols % 16 != 0) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    MOE_TRY(need(src));
    MOE_TRY(need(codes));
    MOE_TRY(need(exps));
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    MOE_LAUNCH(launch_quant_rows_fp8(src, rows, cols, codes, exps, s));
    return MOE_OK;
}

moe_status_t moe_quantize_weights_fp8(const moe_problem_t* p, const void* w_gate, const void* w_up,
                                      const void* w_down, const moe_fp8_weights_t* out, void* stream) {
    MOE_TRY(check_problem(p));
    MOE_TRY(check_fp8(p));
    if (out == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(need(w_gate));
    MOE_TRY(need(w_up));
    MOE_TRY(need(w_down));
    MOE_TRY(need(out->w_gate));
    MOE_TRY(need(out->w_gate_exp));
    MOE_TRY(need(out->w_up));
    MOE_TRY(need(out->w_up_exp));
    MOE_TRY(need(out->w_down));
    MOE_TRY(need(out->w_down_exp));
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    const int64_t ef = static_cast<int64_t>(p->E) * p->f, ed = static_cast<int64_t>(p->E) * p->d;
    MOE_LAUNCH(launch_quant_rows_fp8(w_gate, ef, p->d, out->w_gate, out->w_gate_exp, s));
    MOE_LAUNCH(launch_quant_rows_fp8(w_up, ef, p->d, out->w_up, out->w_up_exp, s));
    MOE_LAUNCH(launch_quant_rows_fp8(w_down, ed, p->f, out->w_down, out->w_down_exp, s));
    return MOE_OK;
}

moe_status_t moe_expert_ffn_fp8(const moe_problem_t* p, const void* x, const int32_t* sorted_assign,
                                const int32_t* offsets, const moe_fp8_weights_t* w, void* y_perm, void* ws,
                                size_t ws_bytes, void* stream) {
    MOE_TRY(check_problem(p));
    MOE_TRY(check_fp8(p));
    if (w == nullptr) return MOE_ERR_INVALID_ARGUMENT;
    if (p->T == 0) return MOE_OK;
    MOE_TRY(need(x));
    MOE_TRY(need(sorted_assign));
    MOE_TRY(need(offsets));
    MOE_TRY(need(w->w_gate));
    MOE_TRY(need(w->w_gate_exp));
    MOE_TRY(need(w->w_up));
    MOE_TRY(need(w->w_up_exp));
    MOE_TRY(need(w->w_down));
    MOE_TRY(need(w->w_down_exp));
    MOE_TRY(need(y_perm));
    MOE_TRY(need(ws));
    if (ws_bytes < ffn_fp8_ws(*p)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    const size_t n = static_cast<size_t>(p->T) * p->k;
    Carver c(ws);
    void* x_q = c.take<char>(static_cast<size_t>(p->T) * p->d);
    int32_t* x_exp = c.take<int32_t>(static_cast<size_t>(p->T) * 4);
    void* h_q = c.take<char>(n * p->f);
    void* h_sc = c.take<char>(n * (p->f / 32));
    float* part = fp8_split_bytes(*p) > 0 ? c.take<float>(fp8_split_bytes(*p)) : nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    clear_hip_error();
    MOE_LAUNCH(launch_quant_rows_fp8(x, p->T, p->d, x_q, x_exp, s));
    MOE_LAUNCH(launch_expert_ffn_fp8(*p, x_q, x_exp, sorted_assign, offsets, w->w_gate, w->w_gate_exp, w->w_up,
                                     w->w_up_exp, w->w_down, w->w_down_exp, h_q, h_sc, part, y_perm, s));
    return MOE_OK;
}

moe_status_t moe_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes % 16 != 0) return MOE_ERR_UNSUPPORTED;
    if (bytes == 0) return MOE_OK;
    MOE_TRY(need(src));
    MOE_TRY(need(dst));
    clear_hip_error();
    MOE_LAUNCH(launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

moe_status_t moe_mfma_peak(int32_t workgroups, int32_t iters, float* sink, void* stream) {
    if (workgroups <= 0 || iters <= 0) return MOE_ERR_INVALID_ARGUMENT;
    MOE_TRY(need(sink));
    clear_hip_error();
    MOE_LAUNCH(launch_mfma_peak(workgroups, iters, sink, static_cast<hipStream_t>(stream)));
    return MOE_OK;
}

}  // extern "C"
