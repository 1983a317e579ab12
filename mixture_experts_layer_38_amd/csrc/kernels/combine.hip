// Combine, aux loss and bias update.
//  combine: MoE notes (www.cf-1.com/news/5905749) §2 step 4 and §2.3 -- the
//           output is the routing-weighted sum of the chosen experts' outputs,
//           put back in token order; 16-byte vectors, k in ascending order,
//           fp32 accumulation.
//  aux:     same notes §1.2, aux = E * sum_e f_e P_e.
//  bias:    engineering page (ybb.press/quantum-computing/18594) §1.2, one
//           +-alpha step toward the average load T*K/E.
#include "../device_common.h"
#include "../launch.h"

namespace moe {

// One thread per 16-byte vector of one output row: thread i handles token
// i / (d / VEC), columns VEC * (i % (d / VEC)) ..; all loads of a thread are
// independent, so short and long token counts both fill the chip.
template <typename T>
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
    for (int k = 0; k < K; ++k) {
        const int r = assign_row[(size_t)t * K + k];
        if ((unsigned)r >= (unsigned)(n_tok * K)) continue;  // dropped (-1)
        const float wk = w[(size_t)t * K + k];
        const u32x4 raw = load16(h + (size_t)r * d + c);
        const T* v = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int j = 0; j < VEC; ++j) acc[j] = fmaf(wk, to_f32(v[j]), acc[j]);
    }
    u32x4 outv;
    T* o = reinterpret_cast<T*>(&outv);
#pragma unroll
    for (int j = 0; j < VEC; ++j) o[j] = from_f32<T>(acc[j]);
    store16(y + (size_t)t * d + c, outv);
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
                         combine_kernel<float><<<grid, 256, 0, s>>>(T, K, d, (const float*)h,
                                                                    assign_row, w, (float*)y));
    else
        MOE_TIMED_LAUNCH(MOE_KERNEL_COMBINE, s,
                         combine_kernel<bf16><<<grid, 256, 0, s>>>(T, K, d, (const bf16*)h,
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
