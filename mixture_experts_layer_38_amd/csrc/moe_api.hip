// C ABI of the MoE layer (include/moe.h): argument checks, workspace layout,
// and the order of launches.  Never allocates, never synchronises.
#include <algorithm>
#include <atomic>
#include <hip/hip_runtime.h>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include "launch.h"

namespace moe {

// ---- timing hook --------------------------------------------------------------
// Process-wide tracing state.  While no timer is armed, a launch reads one
// atomic and touches nothing else, so concurrent layer calls share no
// mutable state; an armed timer's slots are updated under a mutex.
namespace {
struct TimerSlot {
    void* const* start = nullptr;
    void* const* stop = nullptr;
    int n = 0;
    int recorded = 0;
};
TimerSlot g_timer[MOE_KERNEL_COUNT];
std::atomic<int> g_timer_armed{0};  // slots with n > 0
std::mutex g_timer_mu;
}  // namespace

void timer_before(int kid, hipStream_t s) {
    if (g_timer_armed.load(std::memory_order_acquire) == 0) return;
    std::lock_guard<std::mutex> lk(g_timer_mu);
    TimerSlot& t = g_timer[kid];
    if (t.recorded < t.n) (void)hipEventRecord((hipEvent_t)t.start[t.recorded], s);
}
void timer_after(int kid, hipStream_t s) {
    if (g_timer_armed.load(std::memory_order_acquire) == 0) return;
    std::lock_guard<std::mutex> lk(g_timer_mu);
    TimerSlot& t = g_timer[kid];
    if (t.recorded < t.n) {
        (void)hipEventRecord((hipEvent_t)t.stop[t.recorded], s);
        ++t.recorded;
    }
}

// ---- checks --------------------------------------------------------------------
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static moe_status check_problem(const moe_problem* p) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (p->T <= 0 || p->d_model <= 0 || p->n_experts <= 0 || p->top_k <= 0 || p->d_ff <= 0)
        return MOE_ERR_INVALID_ARG;
    if (p->top_k > p->n_experts) return MOE_ERR_INVALID_ARG;
    if (p->flags & ~(uint32_t)(MOE_FLAG_BIAS_SELECT_ONLY | MOE_FLAG_COMBINE_MEAN)) return MOE_ERR_INVALID_ARG;
    if (p->dtype != MOE_DTYPE_F32 && p->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
    if (p->n_experts > 1024 || p->top_k > 32) return MOE_ERR_UNSUPPORTED;
    if (p->d_model % 8 != 0 || p->d_ff % 8 != 0) return MOE_ERR_UNSUPPORTED;
    if (p->d_model > 65536 || p->d_ff > 65536) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)p->T * p->top_k >= (1LL << 30)) return MOE_ERR_UNSUPPORTED;
    // the fp32 kernels run one wave per output element: keep their grids in range
    if (p->dtype == MOE_DTYPE_F32 &&
        ((int64_t)p->T * p->top_k * std::max(p->d_model, p->d_ff) > (1LL << 31) ||
         (int64_t)p->T * p->n_experts > (1LL << 31)))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

#define REQUIRE(ptr)                                      \
    do {                                                  \
        if (!(ptr)) return MOE_ERR_INVALID_ARG;           \
        if (!aligned16(ptr)) return MOE_ERR_ALIGNMENT;    \
    } while (0)
#define OPTIONAL(ptr)                                                 \
    do {                                                              \
        if ((ptr) && !aligned16(ptr)) return MOE_ERR_ALIGNMENT;       \
    } while (0)

static moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

static size_t elem_bytes(const moe_problem* p) { return p->dtype == MOE_DTYPE_F32 ? 4 : 2; }

// ---- workspace layout of moe_forward ------------------------------------------------
struct ForwardLayout {
    size_t logits, probs, prob_sum, ids, w, counts, kept, offsets, assign_row, row_assign;
    size_t act, h, route_ws, disp_ws, ffn_ws, loss_part, total;
};

static ForwardLayout forward_layout(const moe_problem* p) {
    const size_t T = p->T, E = p->n_experts, K = p->top_k, d = p->d_model, F = p->d_ff;
    const size_t n = T * K, es = elem_bytes(p);
    ForwardLayout L;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o += align_up(bytes ? bytes : 1, 256);
        return at;
    };
    L.logits = take(T * E * 4);
    L.probs = take(T * E * 4);
    L.prob_sum = take(E * 4);
    L.ids = take(n * 4);
    L.w = take(n * 4);
    L.counts = take(E * 4);
    L.kept = take(E * 4);
    L.offsets = take((E + 1) * 4);
    L.assign_row = take(n * 4);
    L.row_assign = take(n * 4);
    L.act = take(n * F * es);
    L.h = take(n * d * es);
    L.route_ws = take(std::max(router_ws_bytes(p->T, p->d_model, p->n_experts, p->dtype),
                               route_dispatch_small_ws_bytes(p->T, p->n_experts)));
    L.disp_ws = take(dispatch_ws_bytes(p->T, p->top_k, p->n_experts));
    L.ffn_ws = take(ffn_ws_bytes(p->T, p->top_k, p->n_experts, p->d_model, p->d_ff, p->dtype));
    L.loss_part = take(router_losses_part_bytes(router_num_blocks(p->T, p->n_experts), (int)E));
    L.total = o;
    return L;
}

// Workspace of the chunked forward: the larger of the layouts of the two chunk
// sizes it uses (a full chunk and the remainder; some scratch regions are not
// monotone in T).
static size_t chunked_ws_bytes(const moe_problem* p, int chunk_tokens) {
    moe_problem c = *p;
    c.T = chunk_tokens < p->T ? chunk_tokens : p->T;
    size_t total = forward_layout(&c).total;
    const int rem = p->T % c.T;
    if (rem) {
        c.T = rem;
        const size_t r = forward_layout(&c).total;
        if (r > total) total = r;
    }
    return total;
}

static moe_status check_debug(const moe_debug_out& D) {
    OPTIONAL(D.logits);
    OPTIONAL(D.probs);
    OPTIONAL(D.prob_sum);
    OPTIONAL(D.topk_ids);
    OPTIONAL(D.topk_w);
    OPTIONAL(D.counts);
    OPTIONAL(D.kept);
    OPTIONAL(D.offsets);
    OPTIONAL(D.assign_row);
    OPTIONAL(D.row_assign);
    if ((D.z_loss && ((uintptr_t)D.z_loss & 3u)) || (D.aux_topk && ((uintptr_t)D.aux_topk & 3u)))
        return MOE_ERR_ALIGNMENT;
    return MOE_OK;
}

// The launches of one forward pass over the problem's T tokens, with the
// workspace carved by L (arguments already checked).
static moe_status forward_launch(const moe_problem* p, const ForwardLayout& L, const void* x,
                                 const void* w_router, const void* w1, const void* w3,
                                 const void* w2, const float* logit_bias, void* y,
                                 const moe_debug_out& D, char* base, hipStream_t s) {
    float* logits = D.logits ? D.logits : (float*)(base + L.logits);
    int32_t* ids = D.topk_ids ? D.topk_ids : (int32_t*)(base + L.ids);
    float* w = D.topk_w ? D.topk_w : (float*)(base + L.w);
    int32_t* counts = D.counts ? D.counts : (int32_t*)(base + L.counts);
    int32_t* kept = D.kept ? D.kept : (int32_t*)(base + L.kept);
    int32_t* offsets = D.offsets ? D.offsets : (int32_t*)(base + L.offsets);
    int32_t* assign_row = D.assign_row ? D.assign_row : (int32_t*)(base + L.assign_row);
    int32_t* row_assign = D.row_assign ? D.row_assign : (int32_t*)(base + L.row_assign);
    void* act = base + L.act;
    void* h = base + L.h;
    hipError_t err;
    const bool losses = D.z_loss || D.aux_topk;
    if (route_dispatch_small_ok(p->T, p->d_model, p->n_experts, p->top_k, p->dtype)) {
        // routing, dispatch and the router regularisers in one block
        err = launch_route_dispatch_small(p->T, p->d_model, p->n_experts, p->top_k, (int)p->flags,
                                          p->capacity, x, w_router, logit_bias, logits, D.probs,
                                          D.prob_sum, ids, w, counts, kept, offsets, assign_row,
                                          row_assign, D.z_loss, D.aux_topk, base + L.route_ws, s);
        if (err != hipSuccess) return MOE_ERR_HIP;
    } else {
        float* loss_part = losses ? (float*)(base + L.loss_part) : nullptr;
        err = launch_router(p->T, p->d_model, p->n_experts, p->top_k, p->dtype, (int)p->flags, x,
                            w_router, logit_bias, logits, D.probs, D.prob_sum, ids, w,
                            base + L.route_ws, s, loss_part);
        if (err != hipSuccess) return MOE_ERR_HIP;
        // The grouped token rows are never materialised: the first GEMM reads
        // token row_assign[r] / K for its grouped row r.
        err = launch_dispatch(p->T, p->top_k, p->n_experts, p->d_model, p->dtype, p->capacity, ids,
                              nullptr, counts, kept, offsets, assign_row, row_assign, nullptr,
                              base + L.disp_ws, s);
        if (err != hipSuccess) return MOE_ERR_HIP;
        if (losses) {
            err = launch_router_losses_reduce(p->T, p->n_experts, p->top_k, router_num_blocks(p->T, p->n_experts),
                                              loss_part, counts, D.z_loss, D.aux_topk, s);
            if (err != hipSuccess) return MOE_ERR_HIP;
        }
    }
    err = launch_ffn(p->T, p->top_k, p->n_experts, p->d_model, p->d_ff, p->dtype, x, row_assign,
                     offsets, w1, w3, w2, act, h, base + L.ffn_ws, s);
    if (err != hipSuccess) return MOE_ERR_HIP;
    err = launch_combine(p->T, p->top_k, p->d_model, p->dtype, h, assign_row, w, y, s);
    return hip_status(err);
}

// ---- allocation-free forward ------------------------------------------------------
// The workspace of moe_forward_noalloc: a file-scope device array, one copy
// per GPU the library runs on (held until the process ends).  Host code never
// uses its name as an address: the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_WS_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

// Device address of the current device's copy of `scratch`.
static hipError_t device_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    *out = g_scratch_ptr[dev];
    return g_scratch_err[dev];
}

}  // namespace moe

using namespace moe;

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported problem";
        case MOE_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* moe_version(void) { return "moe-gfx950 0.1"; }

const char* moe_kernel_name(int kid) {
    static const char* names[MOE_KERNEL_COUNT] = {
        "router", "dispatch_count", "dispatch_scan", "dispatch_scatter", "dispatch_gather",
        "ffn_gate_up", "ffn_down", "combine", "aux_loss", "bias_update", "ffn_plan",
        "router_losses", "ffn"};
    return (kid >= 0 && kid < MOE_KERNEL_COUNT) ? names[kid] : "?";
}

moe_status moe_set_kernel_timer(int kid, void* const* start_events, void* const* stop_events,
                                int n_events, int* recorded) {
    if (kid < 0 || kid >= MOE_KERNEL_COUNT) return MOE_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_timer_mu);
    TimerSlot& t = g_timer[kid];
    if (n_events < 0) {
        if (recorded) *recorded = t.recorded;
        return MOE_OK;
    }
    if (n_events > 0 && (!start_events || !stop_events)) return MOE_ERR_INVALID_ARG;
    const bool was = t.n > 0, now = n_events > 0;
    t.start = start_events;
    t.stop = stop_events;
    t.n = n_events;
    t.recorded = 0;
    if (now != was) g_timer_armed.fetch_add(now ? 1 : -1, std::memory_order_release);
    if (recorded) *recorded = 0;
    return MOE_OK;
}

moe_status moe_route_workspace_size(const moe_problem* p, size_t* bytes) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = router_ws_bytes(p->T, p->d_model, p->n_experts, p->dtype);
    return MOE_OK;
}

moe_status moe_dispatch_workspace_size(const moe_problem* p, size_t* bytes) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = dispatch_ws_bytes(p->T, p->top_k, p->n_experts);
    return MOE_OK;
}

moe_status moe_expert_ffn_workspace_size(const moe_problem* p, size_t* bytes) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = ffn_ws_bytes(p->T, p->top_k, p->n_experts, p->d_model, p->d_ff, p->dtype);
    return MOE_OK;
}

moe_status moe_workspace_size(const moe_problem* p, size_t* bytes) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = forward_layout(p).total;
    return MOE_OK;
}

moe_status moe_route(const moe_problem* p, const void* x, const void* w_router,
                     const float* logit_bias, float* logits, float* probs, float* prob_sum,
                     int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    OPTIONAL(x);
    if (x) REQUIRE(w_router);
    REQUIRE(logits);
    REQUIRE(topk_ids);
    REQUIRE(topk_w);
    OPTIONAL(logit_bias);
    OPTIONAL(probs);
    OPTIONAL(prob_sum);
    if (prob_sum || (x && p->dtype == MOE_DTYPE_BF16)) {
        if (!ws || ws_bytes < router_ws_bytes(p->T, p->d_model, p->n_experts, p->dtype))
            return MOE_ERR_WORKSPACE;
        if (!aligned16(ws)) return MOE_ERR_ALIGNMENT;
    }
    return hip_status(launch_router(p->T, p->d_model, p->n_experts, p->top_k, p->dtype, (int)p->flags, x,
                                    w_router, logit_bias, logits, probs, prob_sum, topk_ids,
                                    topk_w, ws, (hipStream_t)stream));
}

moe_status moe_dispatch(const moe_problem* p, const int32_t* topk_ids, const void* x,
                        int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* assign_row,
                        int32_t* row_assign, void* x_perm, void* ws, size_t ws_bytes,
                        void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    REQUIRE(topk_ids);
    REQUIRE(counts);
    REQUIRE(kept);
    REQUIRE(offsets);
    REQUIRE(assign_row);
    REQUIRE(row_assign);
    OPTIONAL(x);
    if (x) REQUIRE(x_perm);
    if (!ws || ws_bytes < dispatch_ws_bytes(p->T, p->top_k, p->n_experts)) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_dispatch(p->T, p->top_k, p->n_experts, p->d_model, p->dtype,
                                      p->capacity, topk_ids, x, counts, kept, offsets, assign_row,
                                      row_assign, x_perm, ws, (hipStream_t)stream));
}

moe_status moe_expert_ffn(const moe_problem* p, const void* x_perm, const int32_t* offsets,
                          const void* w1, const void* w3, const void* w2, void* act, void* h,
                          void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    REQUIRE(x_perm);
    REQUIRE(offsets);
    REQUIRE(w1);
    REQUIRE(w3);
    REQUIRE(w2);
    REQUIRE(act);
    REQUIRE(h);
    const size_t need = ffn_ws_bytes(p->T, p->top_k, p->n_experts, p->d_model, p->d_ff, p->dtype);
    if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_ffn(p->T, p->top_k, p->n_experts, p->d_model, p->d_ff, p->dtype,
                                 x_perm, nullptr, offsets, w1, w3, w2, act, h, ws,
                                 (hipStream_t)stream));
}

moe_status moe_combine(const moe_problem* p, const void* h, const int32_t* assign_row,
                       const float* topk_w, void* y, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    REQUIRE(h);
    REQUIRE(assign_row);
    REQUIRE(topk_w);
    REQUIRE(y);
    return hip_status(launch_combine(p->T, p->top_k, p->d_model, p->dtype, h, assign_row, topk_w,
                                     y, (hipStream_t)stream));
}

moe_status moe_forward(const moe_problem* p, const void* x, const void* w_router, const void* w1,
                       const void* w3, const void* w2, const float* logit_bias, void* y,
                       const moe_debug_out* dbg, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    REQUIRE(x);
    REQUIRE(w_router);
    REQUIRE(w1);
    REQUIRE(w3);
    REQUIRE(w2);
    REQUIRE(y);
    OPTIONAL(logit_bias);
    moe_debug_out none;
    memset(&none, 0, sizeof none);
    const moe_debug_out& D = dbg ? *dbg : none;
    if ((st = check_debug(D)) != MOE_OK) return st;
    const ForwardLayout L = forward_layout(p);
    if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGNMENT;
    return forward_launch(p, L, x, w_router, w1, w3, w2, logit_bias, y, D, (char*)ws,
                          (hipStream_t)stream);
}

moe_status moe_forward_noalloc(const moe_problem* p, const void* x, const void* w_router, const void* w1,
                               const void* w3, const void* w2, const float* logit_bias, void* y,
                               const moe_debug_out* dbg, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    REQUIRE(x);
    REQUIRE(w_router);
    REQUIRE(w1);
    REQUIRE(w3);
    REQUIRE(w2);
    REQUIRE(y);
    OPTIONAL(logit_bias);
    moe_debug_out none;
    memset(&none, 0, sizeof none);
    const moe_debug_out& D = dbg ? *dbg : none;
    if ((st = check_debug(D)) != MOE_OK) return st;
    const ForwardLayout L = forward_layout(p);
    if (L.total > (size_t)MOE_NOALLOC_WS_BYTES) return MOE_ERR_WORKSPACE;
    void* ws = nullptr;
    if (device_scratch(&ws) != hipSuccess || !ws) return MOE_ERR_HIP;
    return forward_launch(p, L, x, w_router, w1, w3, w2, logit_bias, y, D, (char*)ws, (hipStream_t)stream);
}

moe_status moe_forward_chunked_workspace_size(const moe_problem* p, int32_t chunk_tokens,
                                              size_t* bytes) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!bytes || chunk_tokens <= 0) return MOE_ERR_INVALID_ARG;
    *bytes = chunked_ws_bytes(p, chunk_tokens);
    return MOE_OK;
}

moe_status moe_forward_chunked(const moe_problem* p, int32_t chunk_tokens, const void* x,
                               const void* w_router, const void* w1, const void* w3,
                               const void* w2, const float* logit_bias, void* y,
                               const moe_debug_out* dbg, void* ws, size_t ws_bytes,
                               void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (chunk_tokens <= 0) return MOE_ERR_INVALID_ARG;
    if (p->capacity >= 0) return MOE_ERR_UNSUPPORTED;  // a per-batch cap does not split into chunks
    REQUIRE(x);
    REQUIRE(w_router);
    REQUIRE(w1);
    REQUIRE(w3);
    REQUIRE(w2);
    REQUIRE(y);
    OPTIONAL(logit_bias);
    moe_debug_out none;
    memset(&none, 0, sizeof none);
    const moe_debug_out& D = dbg ? *dbg : none;
    if ((st = check_debug(D)) != MOE_OK) return st;
    if (D.prob_sum || D.counts || D.kept || D.offsets || D.assign_row || D.row_assign || D.z_loss ||
        D.aux_topk)
        return MOE_ERR_INVALID_ARG;  // only the per-token outputs are defined across chunks
    const int chunk = chunk_tokens < p->T ? chunk_tokens : p->T;
    moe_problem c = *p;
    if (!ws || ws_bytes < chunked_ws_bytes(p, chunk)) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGNMENT;
    const size_t es = elem_bytes(p);
    const size_t d = p->d_model, E = p->n_experts, K = p->top_k;
    for (int t0 = 0; t0 < p->T; t0 += chunk) {
        c.T = (p->T - t0) < chunk ? (p->T - t0) : chunk;
        const ForwardLayout L = forward_layout(&c);  // within chunked_ws_bytes by construction
        moe_debug_out Dc = D;
        if (D.logits) Dc.logits = D.logits + (size_t)t0 * E;
        if (D.probs) Dc.probs = D.probs + (size_t)t0 * E;
        if (D.topk_ids) Dc.topk_ids = D.topk_ids + (size_t)t0 * K;
        if (D.topk_w) Dc.topk_w = D.topk_w + (size_t)t0 * K;
        st = forward_launch(&c, L, (const char*)x + (size_t)t0 * d * es, w_router, w1, w3, w2,
                            logit_bias, (char*)y + (size_t)t0 * d * es, Dc, (char*)ws,
                            (hipStream_t)stream);
        if (st != MOE_OK) return st;
    }
    return MOE_OK;
}

moe_status moe_aux_loss(const moe_problem* p, const int32_t* counts, const float* prob_sum,
                        float* aux, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!counts || !prob_sum || !aux) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_aux(p->T, p->top_k, p->n_experts, counts, prob_sum, aux,
                                 (hipStream_t)stream));
}

moe_status moe_combine_concat_workspace_size(const moe_problem* p, size_t* bytes) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = combine_concat_ws_bytes(p->T, p->top_k, p->d_model, p->dtype);
    return MOE_OK;
}

moe_status moe_combine_concat(const moe_problem* p, const void* h, const int32_t* assign_row,
                              const void* w_cat, void* y, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    REQUIRE(h);
    REQUIRE(assign_row);
    REQUIRE(w_cat);
    REQUIRE(y);
    if (!ws || ws_bytes < combine_concat_ws_bytes(p->T, p->top_k, p->d_model, p->dtype)) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_combine_concat(p->T, p->top_k, p->d_model, p->dtype, h, assign_row, w_cat, y, ws,
                                            (hipStream_t)stream));
}

moe_status moe_router_losses_workspace_size(const moe_problem* p, size_t* bytes) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!bytes) return MOE_ERR_INVALID_ARG;
    *bytes = router_losses_ws_bytes(p->T, p->n_experts);
    return MOE_OK;
}

moe_status moe_router_losses(const moe_problem* p, const float* logits, const float* logit_bias,
                             const int32_t* topk_ids, const int32_t* counts, float* z_loss,
                             float* aux_topk, void* ws, size_t ws_bytes, void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    REQUIRE(logits);
    REQUIRE(topk_ids);
    OPTIONAL(logit_bias);
    if (!z_loss && !aux_topk) return MOE_ERR_INVALID_ARG;
    if (aux_topk && !counts) return MOE_ERR_INVALID_ARG;
    if (!ws || ws_bytes < router_losses_ws_bytes(p->T, p->n_experts)) return MOE_ERR_WORKSPACE;
    if (!aligned16(ws)) return MOE_ERR_ALIGNMENT;
    return hip_status(launch_router_losses(p->T, p->n_experts, p->top_k, logits, logit_bias,
                                           topk_ids, counts, z_loss, aux_topk, ws,
                                           (hipStream_t)stream));
}

moe_status moe_bias_update(const moe_problem* p, const int32_t* counts, float alpha, float* bias,
                           void* stream) {
    moe_status st = check_problem(p);
    if (st != MOE_OK) return st;
    if (!counts || !bias) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_bias_update(p->T, p->top_k, p->n_experts, counts, alpha, bias,
                                         (hipStream_t)stream));
}

}  // extern "C"
