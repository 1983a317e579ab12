// Grouped expert FFN entry: picks the kernel family for the problem.
//  - bf16 with at most 64 tokens (so at most 64 rows per expert): the
//    weight-streaming decode kernels (ffn_decode.hip);
//  - other bf16 problems: the LDS-tiled MFMA kernels (ffn_prefill.hip);
//  - fp32: plain FMA kernels below (one wave per output element), kept for
//    the small fp32 layer.
#include "../device_common.h"
#include "../launch.h"

namespace moe {

hipError_t launch_ffn_decode(int n_rows, int E, int d, int F, const void* A, const int32_t* rowmap,
                             int topk, const int32_t* offsets, const void* w1, const void* w3,
                             const void* w2, void* act, void* h, hipStream_t s);
hipError_t launch_ffn_prefill(int n_rows, int E, int d, int F, const void* A, const int32_t* rowmap,
                              int topk, const int32_t* offsets, const void* w1, const void* w3,
                              const void* w2, void* act, void* h, void* ws, hipStream_t s);
size_t prefill_ws_bytes(int n_rows, int E, int d);

constexpr int kDecodeMaxTokens = 64;

// Expert owning grouped row `row` (< offsets[E]): the largest e with offsets[e] <= row.
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int row) {
    int lo = 0, hi = E;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= row) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// fp32 kernels: one wave per output element.  Lane l takes k = l, l + 64, ...
// (so each load instruction reads 256 contiguous bytes of the weight row and
// of the token row), then the 64 partial sums meet in a fixed-order butterfly.
__global__ __launch_bounds__(256) void ffn_f32_gate_up_kernel(int n_rows, int E, int F, int d,
                                                             const float* __restrict__ A,
                                                             const int32_t* __restrict__ rowmap, int topk,
                                                             const int32_t* __restrict__ offsets,
                                                             const float* __restrict__ w1,
                                                             const float* __restrict__ w3,
                                                             float* __restrict__ act) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) / kWave;  // output of this wave
    const int lane = lane_id();
    const int S = min(offsets[E], n_rows);
    if (i >= (size_t)S * F) return;
    const int row = (int)(i / F);
    const int f = (int)(i - (size_t)row * F);
    const int e = expert_of_row(offsets, E, row);
    const float* a = A + (size_t)src_row(rowmap, topk, row) * d;
    const float* r1 = w1 + ((size_t)e * F + f) * d;
    const float* r3 = w3 + ((size_t)e * F + f) * d;
    float g1 = 0.0f, g3 = 0.0f;
    for (int j = lane; j < d; j += kWave) {
        const float av = a[j];
        g1 = fmaf(r1[j], av, g1);
        g3 = fmaf(r3[j], av, g3);
    }
    g1 = wave_sum(g1);
    g3 = wave_sum(g3);
    if (lane == 0) act[i] = g1 / (1.0f + expf(-g1)) * g3;
}

__global__ __launch_bounds__(256) void ffn_f32_down_kernel(int n_rows, int E, int F, int d,
                                                          const float* __restrict__ act,
                                                          const int32_t* __restrict__ offsets,
                                                          const float* __restrict__ w2,
                                                          float* __restrict__ h) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) / kWave;
    const int lane = lane_id();
    const int S = min(offsets[E], n_rows);
    if (i >= (size_t)S * d) return;
    const int row = (int)(i / d);
    const int c = (int)(i - (size_t)row * d);
    const int e = expert_of_row(offsets, E, row);
    const float* a = act + (size_t)row * F;
    const float* r2 = w2 + ((size_t)e * d + c) * F;
    float sum = 0.0f;
    for (int f = lane; f < F; f += kWave) sum = fmaf(r2[f], a[f], sum);
    sum = wave_sum(sum);
    if (lane == 0) h[i] = sum;
}

static bool use_decode(int T, int dtype) { return dtype == MOE_DTYPE_BF16 && T <= kDecodeMaxTokens; }

size_t ffn_ws_bytes(int T, int K, int E, int d, int /*F*/, int dtype) {
    if (dtype != MOE_DTYPE_BF16 || use_decode(T, dtype)) return 256;
    return prefill_ws_bytes(T * K, E, d);
}

static hipError_t launch_ffn_paths(int T, int K, int E, int d, int F, int dtype, const void* A,
                                   const int32_t* rowmap, const int32_t* offsets, const void* w1,
                                   const void* w3, const void* w2, void* act, void* h, void* ws,
                                   hipStream_t s) {
    const int n = T * K;
    if (dtype == MOE_DTYPE_F32) {
        const size_t n1 = (size_t)n * F, n2 = (size_t)n * d;
        // one wave (a quarter of a 256-thread block) per output element
        MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_GATE_UP, s,
                         ffn_f32_gate_up_kernel<<<(unsigned)((n1 + 3) / 4), 256, 0, s>>>(
                             n, E, F, d, (const float*)A, rowmap, K, offsets, (const float*)w1,
                             (const float*)w3, (float*)act));
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_DOWN, s,
                         ffn_f32_down_kernel<<<(unsigned)((n2 + 3) / 4), 256, 0, s>>>(
                             n, E, F, d, (const float*)act, offsets, (const float*)w2, (float*)h));
        return hipGetLastError();
    }
    if (use_decode(T, dtype))
        return launch_ffn_decode(n, E, d, F, A, rowmap, K, offsets, w1, w3, w2, act, h, s);
    return launch_ffn_prefill(n, E, d, F, A, rowmap, K, offsets, w1, w3, w2, act, h, ws, s);
}

// The expert FFN as one timed step (MOE_KERNEL_FFN): every launch of both GEMMs.
hipError_t launch_ffn(int T, int K, int E, int d, int F, int dtype, const void* A,
                      const int32_t* rowmap, const int32_t* offsets, const void* w1,
                      const void* w3, const void* w2, void* act, void* h, void* ws, hipStream_t s) {
    timer_before(MOE_KERNEL_FFN, s);
    const hipError_t err = launch_ffn_paths(T, K, E, d, F, dtype, A, rowmap, offsets, w1, w3, w2, act, h, ws, s);
    if (err == hipSuccess) timer_after(MOE_KERNEL_FFN, s);
    return err;
}

}  // namespace moe
