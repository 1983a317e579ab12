// Host-side launch wrappers of the MoE kernels (internal to libmoe.so).
// Shapes have been validated by the C ABI layer before any of these runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ---- kernel timing hook ----------------------------------------------------
void timer_before(int kid, hipStream_t s);
void timer_after(int kid, hipStream_t s);

// Launch `expr` (a kernel launch) bracketed by the timing hook of kernel `kid`.
#define MOE_TIMED_LAUNCH(kid, stream, ...)        \
    do {                                          \
        ::moe::timer_before((kid), (stream));     \
        __VA_ARGS__;                              \
        ::moe::timer_after((kid), (stream));      \
    } while (0)

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---- router ----------------------------------------------------------------
// Number of token blocks of the route kernel (its prob_sum partials are per block).
int router_num_blocks(int T, int E);
// Workspace of the router: W_r^T and partial scores (bf16 scores from x) and
// the per-block probability sums.
size_t router_ws_bytes(int T, int d, int E, int dtype);
// loss_part (optional, router_losses_part_bytes(router_num_blocks(T, E), E)
// bytes): the route kernel's per-block partials of the router regularisers
// (the first router_num_blocks(T, E) * (E + 1) floats), for
// launch_router_losses_reduce.
hipError_t launch_router(int T, int d, int E, int K, int dtype, int flags, const void* x,
                         const void* w_router, const float* bias, float* logits, float* probs,
                         float* prob_sum, int32_t* ids, float* w, void* ws, hipStream_t s,
                         float* loss_part = nullptr);

// Small batches (bf16, T <= 64, E <= 16): scores, routing and dispatch in two
// launches, with the outputs of launch_router followed by launch_dispatch
// (x == NULL there).  ws: route_dispatch_small_ws_bytes.
bool route_dispatch_small_ok(int T, int d, int E, int K, int dtype);
size_t route_dispatch_small_ws_bytes(int T, int E);
hipError_t launch_route_dispatch_small(int T, int d, int E, int K, int flags, int capacity, const void* x,
                                       const void* w_router, const float* bias, float* logits,
                                       float* probs, float* prob_sum, int32_t* ids, float* w,
                                       int32_t* counts, int32_t* kept, int32_t* offsets,
                                       int32_t* assign_row, int32_t* row_assign, float* z_loss,
                                       float* aux_topk, void* ws, hipStream_t s);
// ---- dispatch --------------------------------------------------------------
size_t dispatch_ws_bytes(int T, int K, int E);
hipError_t launch_dispatch(int T, int K, int E, int d, int dtype, int capacity,
                           const int32_t* ids, const void* x, int32_t* counts, int32_t* kept,
                           int32_t* offsets, int32_t* assign_row, int32_t* row_assign,
                           void* x_perm, void* ws, hipStream_t s);

// ---- grouped expert FFN ----------------------------------------------------
size_t ffn_ws_bytes(int T, int K, int E, int d, int F, int dtype);
// A: the grouped rows [T*K, d] when rowmap is NULL; otherwise the token rows
// x [T, d], and grouped row r reads token rowmap[r] / K (rowmap = row_assign
// of the dispatch; -1 past the kept rows reads token 0, whose results are
// never stored).
hipError_t launch_ffn(int T, int K, int E, int d, int F, int dtype, const void* A,
                      const int32_t* rowmap, const int32_t* offsets, const void* w1,
                      const void* w3, const void* w2, void* act, void* h, void* ws, hipStream_t s);

// Inside a large batch, the experts with at most DC_SMALL_ROWS rows run on
// the weight-streaming decode kernel (the tiled GEMM skips them).
constexpr int DC_SMALL_ROWS = 32;
// elist[0 .. *ecount): the small experts (device memory, written by the tile plan).
hipError_t launch_small_experts(bool gated, int E, int n_rows, int N, int K, const void* A,
                                const int32_t* rowmap, int topk, const int32_t* offsets, const int32_t* elist,
                                const int32_t* ecount, const void* wa, const void* wb, void* out, hipStream_t s);
// ---- router regularisers ----------------------------------------------------
size_t router_losses_ws_bytes(int T, int E);
// Bytes of a partials buffer for nblk blocks: the partials themselves
// ([nblk][E] chosen-probability sums, then [nblk] squared log-sum-exps), then
// room for the reduce's second-level sums.
size_t router_losses_part_bytes(int nblk, int E);
// The final sums of the regularisers from nblk blocks of partials in part
// (router_losses_part_bytes(nblk, E) bytes).
hipError_t launch_router_losses_reduce(int T, int E, int K, int nblk, float* part, const int32_t* counts,
                                       float* z_loss, float* aux_topk, hipStream_t s);
hipError_t launch_router_losses(int T, int E, int K, const float* logits, const float* bias,
                                const int32_t* ids, const int32_t* counts, float* z_loss,
                                float* aux_topk, void* ws, hipStream_t s);

// ---- linear layer on the expert-GEMM kernels ---------------------------------
// y[t, o] = sum_j x[t, j] * W[o, j] for t < n_rows (bf16, fp32 accumulation):
// x [n_rows, K], W [N, K], y [n_rows, N]; offs = {0, n_rows} in device memory
// (the kernels see one group of rows).  Small n_rows stream W once through the
// decode kernel (its reduction split into parts when W has few rows), larger
// ones use the tiled GEMM.  ws: linear_ws_bytes, 256-byte aligned.
size_t linear_ws_bytes(int n_rows, int N, int K);
constexpr int LIN_SMALL_ROWS = 64;
constexpr int LIN_MAX_PARTS = 8;
size_t linear_small_ws_bytes(int n_rows, int N, int K);
hipError_t launch_linear_small(int n_rows, int N, int K, const void* A, const int32_t* offs, const void* w,
                               void* out, void* ws, hipStream_t s);
hipError_t launch_linear(int n_rows, int N, int K, const void* x, const int32_t* offs, const void* w,
                         void* y, void* ws, hipStream_t s);
// Concatenation combine for at most LIN_SMALL_ROWS tokens (bf16): the
// weight-streaming kernel reads each slot's grouped rows h[assign_row[t,k]]
// in place, its reduction split into parts that never straddle a slot.
// concat_small_ok says whether this path applies; ws: concat_small_ws_bytes.
bool concat_small_ok(int T, int Ks, int d);
size_t concat_small_ws_bytes(int T, int Ks, int d);
hipError_t launch_concat_small(int T, int Ks, int d, const void* h, const int32_t* assign_row, const void* w_cat,
                               void* y, void* ws, hipStream_t s);
// ---- combine / aux / bias --------------------------------------------------
// Concatenation combine: y[t] = W_cat . concat over slots of h[assign_row[t,k]].
size_t combine_concat_ws_bytes(int T, int K, int d, int dtype);
hipError_t launch_combine_concat(int T, int K, int d, int dtype, const void* h, const int32_t* assign_row,
                                 const void* w_cat, void* y, void* ws, hipStream_t s);
hipError_t launch_combine(int T, int K, int d, int dtype, const void* h,
                          const int32_t* assign_row, const float* w, void* y, hipStream_t s);
hipError_t launch_aux(int T, int K, int E, const int32_t* counts, const float* prob_sum,
                      float* aux, hipStream_t s);
hipError_t launch_bias_update(int T, int K, int E, const int32_t* counts, float alpha,
                              float* bias, hipStream_t s);

}  // namespace moe
