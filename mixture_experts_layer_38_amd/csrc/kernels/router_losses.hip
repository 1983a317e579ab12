// Router regularisers of the MoE notes (www.cf-1.com/news/5905749) §3.2:
//   z_loss   = (1/T) sum_t (log sum_e exp(logits[t,e]))^2, on the router
//              scores before the per-expert bias;
//   aux_topk = E sum_e f_e P'_e, the cheaper aux loss that keeps only the
//              routing probability of each token's chosen experts:
//              f_e = counts[e] / (T K), P'_e = (1/T) sum_t sum_k [ids[t,k] = e] p[t,e],
//              p = softmax over all E of logits + bias (the routing softmax).
// Two kernels, no atomics: per-token work writes per-block partial sums (a
// wave per token, 16 tokens per block, fixed order inside the block), then one
// block reduces the partials in a fixed order in double.  Inside the layer the
// route kernel writes the same partials from its own softmax (one pass over
// the scores), and only the reduce kernel runs here.
#include <math.h>

#include "../device_common.h"
#include "../launch.h"

namespace moe {

constexpr int RL_BT = 16;  // tokens per block (four per wave)
constexpr int RL_WAVES = 4;

int router_losses_blocks(int T) { return (T + RL_BT - 1) / RL_BT; }

size_t router_losses_ws_bytes(int T, int E) {
    return align_up((size_t)router_losses_blocks(T) * (E + 1) * sizeof(float), 256);
}

// part: [nblk][E] chosen-probability sums, then [nblk] sums of lse^2.
template <int MAXV>
__global__ __launch_bounds__(RL_WAVES * kWave) void router_losses_kernel(
    int T, int E, int K, const float* __restrict__ logits, const float* __restrict__ bias,
    const int32_t* __restrict__ ids, float* __restrict__ part) {
    extern __shared__ float red[];  // [RL_WAVES][E] chosen-probability sums, then [RL_WAVES] z sums
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    float* mine = red + wave * E;
    for (int e = lane; e < E; e += kWave) mine[e] = 0.0f;
    float zsum = 0.0f;
    for (int tt = wave; tt < RL_BT; tt += RL_WAVES) {
        const int t = blockIdx.x * RL_BT + tt;
        if (t >= T) break;
        const float* lg = logits + (size_t)t * E;
        float v[MAXV], vb[MAXV];
        float m = -INFINITY, mb = -INFINITY;
#pragma unroll
        for (int j = 0; j < MAXV; ++j) {
            const int e = lane + j * kWave;
            v[j] = e < E ? lg[e] : -INFINITY;
            vb[j] = e < E ? v[j] + (bias ? bias[e] : 0.0f) : -INFINITY;
            m = fmaxf(m, v[j]);
            mb = fmaxf(mb, vb[j]);
        }
        m = wave_max(m);
        mb = wave_max(mb);
        float s = 0.0f, sb = 0.0f;
#pragma unroll
        for (int j = 0; j < MAXV; ++j) {
            const int e = lane + j * kWave;
            if (e < E) {
                s += expf(v[j] - m);
                sb += expf(vb[j] - mb);
            }
        }
        s = wave_sum(s);
        sb = wave_sum(sb);
        const float lse = m + logf(s);
        zsum += lse * lse;
        // lane k adds the routing probability of the token's k-th chosen
        // expert; the K experts of a token are distinct, so the lanes touch
        // distinct entries, and the wave's tokens follow one another in order.
        if (lane < K) {
            const int e = ids[(size_t)t * K + lane];
            if ((unsigned)e < (unsigned)E) {
                const float lb = lg[e] + (bias ? bias[e] : 0.0f);
                mine[e] += expf(lb - mb) / sb;
            }
        }
    }
    float* zred = red + RL_WAVES * E;
    if (lane == 0) zred[wave] = zsum;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += RL_WAVES * kWave) {
        float acc = red[e];
        for (int w = 1; w < RL_WAVES; ++w) acc += red[w * E + e];
        part[(size_t)blockIdx.x * E + e] = acc;
    }
    if (threadIdx.x == 0) {
        float acc = zred[0];
        for (int w = 1; w < RL_WAVES; ++w) acc += zred[w];
        part[(size_t)gridDim.x * E + blockIdx.x] = acc;
    }
}

// One block of 1024 threads: wave w reduces experts w, w + 16, ... (lanes over
// blocks, then a fixed butterfly), then thread 0 forms both losses in order.
__global__ __launch_bounds__(1024) void router_losses_reduce_kernel(
    int T, int E, int K, int nblk, const float* __restrict__ part, const int32_t* __restrict__ counts,
    float* __restrict__ z_loss, float* __restrict__ aux_topk) {
    __shared__ double pe[1024];
    __shared__ double zs;
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    for (int e = wave; e < E; e += 1024 / kWave) {
        double s = 0.0;
        for (int b = lane; b < nblk; b += kWave) s += (double)part[(size_t)b * E + e];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
        if (lane == 0) pe[e] = s;
    }
    if (wave == 1024 / kWave - 1) {
        double s = 0.0;
        for (int b = lane; b < nblk; b += kWave) s += (double)part[(size_t)nblk * E + b];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
        if (lane == 0) zs = s;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        if (z_loss) *z_loss = (float)(zs / (double)T);
        if (aux_topk) {
            double acc = 0.0;
            for (int e = 0; e < E; ++e)
                acc += (double)counts[e] / ((double)T * K) * (pe[e] / (double)T);
            *aux_topk = (float)((double)E * acc);
        }
    }
}

hipError_t launch_router_losses_reduce(int T, int E, int K, int nblk, const float* part, const int32_t* counts,
                                       float* z_loss, float* aux_topk, hipStream_t s) {
    MOE_TIMED_LAUNCH(MOE_KERNEL_ROUTER_LOSSES, s,
                     router_losses_reduce_kernel<<<1, 1024, 0, s>>>(T, E, K, nblk, part, counts, z_loss, aux_topk));
    return hipGetLastError();
}

hipError_t launch_router_losses(int T, int E, int K, const float* logits, const float* bias,
                                const int32_t* ids, const int32_t* counts, float* z_loss,
                                float* aux_topk, void* ws, hipStream_t s) {
    const int nblk = router_losses_blocks(T);
    float* part = reinterpret_cast<float*>(ws);
    const size_t lds = (size_t)(RL_WAVES * E + RL_WAVES) * sizeof(float);
    if (E <= 64)
        MOE_TIMED_LAUNCH(MOE_KERNEL_ROUTER_LOSSES, s,
                         router_losses_kernel<1><<<nblk, RL_WAVES * kWave, lds, s>>>(T, E, K, logits, bias, ids, part));
    else if (E <= 256)
        MOE_TIMED_LAUNCH(MOE_KERNEL_ROUTER_LOSSES, s,
                         router_losses_kernel<4><<<nblk, RL_WAVES * kWave, lds, s>>>(T, E, K, logits, bias, ids, part));
    else
        MOE_TIMED_LAUNCH(MOE_KERNEL_ROUTER_LOSSES, s,
                         router_losses_kernel<16><<<nblk, RL_WAVES * kWave, lds, s>>>(T, E, K, logits, bias, ids, part));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    router_losses_reduce_kernel<<<1, 1024, 0, s>>>(T, E, K, nblk, part, counts, z_loss, aux_topk);
    return hipGetLastError();
}

}  // namespace moe
