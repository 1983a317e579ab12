// Combine, aux loss and bias update.
//  combine: MoE notes (www.cf-1.com/news/5905749) §2 step 4 and §2.3 -- the
//           output is the routing-weighted sum of the chosen experts' outputs,
//           put back in token order; 16-byte vectors, k in ascending order,
//           fp32 accumulation.
//  aux:     same notes §1.2, aux = E * sum_e f_e P_e.
//  bias:    engineering page (ybb.press/quantum-computing/18594) §1.2, one
//           +-alpha step toward the average load T*K/E.
#include <algorithm>

#include "../device_common.h"
#include "../launch.h"

namespace moe {

// One thread per 16-byte vector of one output row: thread i handles token
// i / (d / VEC), columns VEC * (i % (d / VEC)) ..; all loads of a thread are
// independent, so short and long token counts both fill the chip.
template <typename T, int KC>
__global__ __launch_bounds__(256) void combine_kernel(int n_tok, int K, int d,
                                                     const T* __restrict__ h,
                                                     const int32_t* __restrict__ assign_row,
                                                     const float* __restrict__ w,
                                                     T* __restrict__ y) {
    constexpr int VEC = 16 / sizeof(T);
    const int per_tok = d / VEC;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)n_tok * per_tok) return;
    const int t = (int)(i / per_tok);
    const int c = (int)(i - (size_t)t * per_tok) * VEC;
    float acc[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) acc[j] = 0.0f;
    // Slots in chunks of KC: the chunk's row indices and weights, then all of
    // its rows' loads, then the sums in slot order (so the result does not
    // depend on KC).
    for (int k0 = 0; k0 < K; k0 += KC) {
        int r[KC];
        float wk[KC];
#pragma unroll
        for (int q = 0; q < KC; ++q) {
            const bool in = k0 + q < K;
            r[q] = in ? assign_row[(size_t)t * K + k0 + q] : -1;
            wk[q] = in ? w[(size_t)t * K + k0 + q] : 0.0f;
        }
        u32x4 raw[KC];
#pragma unroll
        for (int q = 0; q < KC; ++q) {
            const bool ok = (unsigned)r[q] < (unsigned)(n_tok * K);  // dropped slot: -1
            raw[q] = load16_or_zero(h + (size_t)(ok ? r[q] : 0) * d + c, ok);
        }
#pragma unroll
        for (int q = 0; q < KC; ++q) {
            if ((unsigned)r[q] >= (unsigned)(n_tok * K)) continue;
            const T* v = reinterpret_cast<const T*>(&raw[q]);
#pragma unroll
            for (int j = 0; j < VEC; ++j) acc[j] = fmaf(wk[q], to_f32(v[j]), acc[j]);
        }
    }
    u32x4 outv;
    T* o = reinterpret_cast<T*>(&outv);
#pragma unroll
    for (int j = 0; j < VEC; ++j) o[j] = from_f32<T>(acc[j]);
    store16(y + (size_t)t * d + c, outv);
}

// Concatenation combine, first half: X[t] = concat over slots k of
// h[assign_row[t,k]] (a zero block for a dropped slot), one thread per 16-byte
// vector; block 0 also writes the one-group row offsets {0, T} that the linear
// layer's GEMM reads.
template <typename T>
__global__ __launch_bounds__(256) void concat_gather_kernel(int n_tok, int K, int d,
                                                           const T* __restrict__ h,
                                                           const int32_t* __restrict__ assign_row,
                                                           T* __restrict__ x, int32_t* __restrict__ offs) {
    constexpr int VEC = 16 / sizeof(T);
    const int per_tok = K * d / VEC;
    if (blockIdx.x == 0 && threadIdx.x < 2) offs[threadIdx.x] = threadIdx.x == 0 ? 0 : n_tok;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)n_tok * per_tok) return;
    const int t = (int)(i / per_tok);
    const int c = (int)(i - (size_t)t * per_tok) * VEC;  // column of X
    const int k = c / d;
    const int r = assign_row[(size_t)t * K + k];
    const u32x4 z = {0u, 0u, 0u, 0u};
    const u32x4 v = (unsigned)r < (unsigned)(n_tok * K) ? load16(h + (size_t)r * d + (c - k * d)) : z;
    store16(x + (size_t)t * K * d + c, v);
}

// fp32 linear layer: y[t, o] = sum_j x[t, j] * W[o, j], one thread per output.
__global__ __launch_bounds__(256) void linear_f32_kernel(int n_tok, int n_out, int n_in,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ w,
                                                        float* __restrict__ y) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)n_tok * n_out) return;
    const int t = (int)(i / n_out);
    const int o = (int)(i - (size_t)t * n_out);
    const float* xr = x + (size_t)t * n_in;
    const float* wr = w + (size_t)o * n_in;
    float s = 0.0f;
    for (int j = 0; j < n_in; ++j) s = fmaf(xr[j], wr[j], s);
    y[i] = s;
}

size_t combine_concat_ws_bytes(int T, int K, int d, int dtype) {
    const size_t es = dtype == MOE_DTYPE_F32 ? 4 : 2;
    size_t b = align_up((size_t)T * K * d * es, 256) + 256;
    if (dtype == MOE_DTYPE_BF16) b += linear_ws_bytes(T, d, K * d);
    if (dtype == MOE_DTYPE_BF16 && concat_small_ok(T, K, d)) b = std::max(b, concat_small_ws_bytes(T, K, d));
    return b;
}

hipError_t launch_combine_concat(int T, int K, int d, int dtype, const void* h, const int32_t* assign_row,
                                 const void* w_cat, void* y, void* ws, hipStream_t s) {
    const size_t es = dtype == MOE_DTYPE_F32 ? 4 : 2;
    char* base = reinterpret_cast<char*>(ws);
    void* x = base;
    int32_t* offs = reinterpret_cast<int32_t*>(base + align_up((size_t)T * K * d * es, 256));
    void* lws = base + align_up((size_t)T * K * d * es, 256) + 256;
    const size_t nvec = (size_t)T * K * d * es / 16;
    const unsigned grid = (unsigned)((nvec + 255) / 256);
    if (dtype == MOE_DTYPE_F32) {
        concat_gather_kernel<float><<<grid, 256, 0, s>>>(T, K, d, (const float*)h, assign_row, (float*)x, offs);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        const size_t n = (size_t)T * d;
        linear_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(T, d, K * d, (const float*)x,
                                                                       (const float*)w_cat, (float*)y);
        return hipGetLastError();
    }
    if (concat_small_ok(T, K, d)) return launch_concat_small(T, K, d, h, assign_row, w_cat, y, ws, s);
    concat_gather_kernel<bf16><<<grid, 256, 0, s>>>(T, K, d, (const bf16*)h, assign_row, (bf16*)x, offs);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_linear(T, d, K * d, x, offs, w_cat, y, lws, s);
}

__global__ __launch_bounds__(1024) void aux_kernel(int T, int K, int E,
                                                  const int32_t* __restrict__ counts,
                                                  const float* __restrict__ prob_sum,
                                                  float* __restrict__ aux) {
    __shared__ double part[1024];
    const int e = threadIdx.x;
    double v = 0.0;
    if (e < E) {
        const double f = (double)counts[e] / ((double)T * K);
        const double P = (double)prob_sum[e] / (double)T;
        v = f * P;
    }
    part[e] = v;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if (e < s) part[e] += part[e + s];
        __syncthreads();
    }
    if (e == 0) *aux = (float)((double)E * part[0]);
}

__global__ __launch_bounds__(256) void bias_update_kernel(int T, int K, int E,
                                                         const int32_t* __restrict__ counts,
                                                         float alpha, float* __restrict__ bias) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    const long long load = (long long)counts[e] * E;
    const long long target = (long long)T * K;
    if (load > target) bias[e] = bias[e] - alpha;
    else if (load < target) bias[e] = bias[e] + alpha;
}

hipError_t launch_combine(int T, int K, int d, int dtype, const void* h,
                          const int32_t* assign_row, const float* w, void* y, hipStream_t s) {
    const size_t vecs = (size_t)T * d / (dtype == MOE_DTYPE_F32 ? 4 : 8);
    const unsigned grid = (unsigned)((vecs + 255) / 256);
    if (dtype == MOE_DTYPE_F32)
        MOE_TIMED_LAUNCH(MOE_KERNEL_COMBINE, s,
                         combine_kernel<float, 2><<<grid, 256, 0, s>>>(T, K, d, (const float*)h,
                                                                       assign_row, w, (float*)y));
    else if (K <= 2)
        MOE_TIMED_LAUNCH(MOE_KERNEL_COMBINE, s,
                         combine_kernel<bf16, 2><<<grid, 256, 0, s>>>(T, K, d, (const bf16*)h,
                                                                      assign_row, w, (bf16*)y));
    else
        MOE_TIMED_LAUNCH(MOE_KERNEL_COMBINE, s,
                         combine_kernel<bf16, 8><<<grid, 256, 0, s>>>(T, K, d, (const bf16*)h,
                                                                      assign_row, w, (bf16*)y));
    return hipGetLastError();
}

hipError_t launch_aux(int T, int K, int E, const int32_t* counts, const float* prob_sum,
                      float* aux, hipStream_t s) {
    MOE_TIMED_LAUNCH(MOE_KERNEL_AUX, s, aux_kernel<<<1, 1024, 0, s>>>(T, K, E, counts, prob_sum, aux));
    return hipGetLastError();
}

hipError_t launch_bias_update(int T, int K, int E, const int32_t* counts, float alpha,
                              float* bias, hipStream_t s) {
    MOE_TIMED_LAUNCH(MOE_KERNEL_BIAS_UPDATE, s,
                     bias_update_kernel<<<(E + 255) / 256, 256, 0, s>>>(T, K, E, counts, alpha, bias));
    return hipGetLastError();
}

}  // namespace moe
