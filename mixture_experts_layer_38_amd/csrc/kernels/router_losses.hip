// Router regularisers of the MoE notes (www.cf-1.com/news/5905749) §3.2:
//   z_loss   = (1/T) sum_t (log sum_e exp(logits[t,e]))^2, on the router
//              scores before the per-expert bias;
//   aux_topk = E sum_e f_e P'_e, the cheaper aux loss that keeps only the
//              routing probability of each token's chosen experts:
//              f_e = counts[e] / (T K), P'_e = (1/T) sum_t sum_k [ids[t,k] = e] p[t,e],
//              p = softmax over all E of logits + bias (the routing softmax).
// No atomics: per-token work writes per-block partial sums (a wave per token,
// 16 tokens per block, fixed order inside the block), then two small launches
// reduce the partials in a fixed order in double.  Inside the layer the
// route kernel writes the same partials from its own softmax (one pass over
// the scores), and only the reduce kernel runs here.
#include <math.h>

#include "../device_common.h"
#include "../launch.h"

namespace moe {

constexpr int RL_BT = 16;  // tokens per block (four per wave)
constexpr int RL_WAVES = 4;

int router_losses_blocks(int T) { return (T + RL_BT - 1) / RL_BT; }

// Second-level partial sums of the reduce: RL_G groups of blocks.
constexpr int RL_G = 64;

size_t router_losses_part_bytes(int nblk, int E) {
    return align_up((size_t)nblk * (E + 1) * sizeof(float), 256) +
           align_up((size_t)RL_G * (E + 1) * sizeof(double), 256);
}

size_t router_losses_ws_bytes(int T, int E) { return router_losses_part_bytes(router_losses_blocks(T), E); }

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

// Reduce of the per-block partials in two launches, in a fixed order and in
// double.  Level 1: workgroup g of G adds blocks [g nblk / G, (g + 1) nblk / G)
// in block order for every column (the E experts' chosen-probability sums,
// then the sum of lse^2), thread c taking columns c, c + 256, ...: consecutive
// threads read consecutive experts of a block, eight loads in flight.
__global__ __launch_bounds__(256) void router_losses_reduce1_kernel(int E, int nblk, int G,
                                                                   const float* __restrict__ part,
                                                                   double* __restrict__ lvl1) {
    const int g = blockIdx.x;
    const int b0 = (int)((long)g * nblk / G), b1 = (int)((long)(g + 1) * nblk / G);
    for (int c = threadIdx.x; c <= E; c += 256) {
        // column c of block b: part[b E + c] for an expert, part[nblk E + b] for lse^2
        const size_t base = c < E ? (size_t)c : (size_t)nblk * E;
        const size_t stride = c < E ? (size_t)E : 1;
        double s = 0.0;
        for (int b = b0; b < b1; b += 8) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = b + q < b1 ? part[base + (size_t)(b + q) * stride] : 0.0f;
#pragma unroll
            for (int q = 0; q < 8; ++q) s += (double)v[q];
        }
        lvl1[(size_t)g * (E + 1) + c] = s;
    }
}

// Level 2, one block of 1024 threads: with R threads per expert (the largest
// power of two with R E <= 1024), thread t adds groups t / E, + R, ... of
// expert t % E, and a fixed pairwise tree adds each expert's R sums; wave 0
// adds the G lse^2 sums with a fixed butterfly.  Then the aux terms
// f_e P'_e go through a fixed pairwise tree, and thread 0 writes both losses.
__global__ __launch_bounds__(1024) void router_losses_reduce2_kernel(
    int T, int E, int K, int G, const double* __restrict__ lvl1, const int32_t* __restrict__ counts,
    float* __restrict__ z_loss, float* __restrict__ aux_topk) {
    __shared__ double red[1024];
    __shared__ double zs;
    const int t = threadIdx.x;
    const int C = E + 1;
    int R = 1;
    while (2 * R * E <= 1024) R *= 2;
    double s = 0.0;
    if (t < R * E) {
        const int e = t % E;
        for (int g = t / E; g < G; g += 8 * R) {
            double v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = g + q * R < G ? lvl1[(size_t)(g + q * R) * C + e] : 0.0;
#pragma unroll
            for (int q = 0; q < 8; ++q) s += v[q];
        }
    }
    red[t] = s;
    if (t < kWave) {
        double z = t < G ? lvl1[(size_t)t * C + E] : 0.0;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
        if (t == 0) zs = z;
    }
    __syncthreads();
    for (int o = R / 2; o > 0; o >>= 1) {
        if (t < o * E) red[t] += red[t + o * E];
        __syncthreads();
    }
    const double term = t < E ? (double)counts[t] / ((double)T * K) * (red[t] / (double)T) : 0.0;
    __syncthreads();
    red[t] = term;
    __syncthreads();
    for (int o = 512; o > 0; o >>= 1) {
        if (t < o) red[t] += red[t + o];
        __syncthreads();
    }
    if (t == 0) {
        if (z_loss) *z_loss = (float)(zs / (double)T);
        if (aux_topk) *aux_topk = (float)((double)E * red[0]);
    }
}

// part: router_losses_part_bytes(nblk, E) bytes, the per-block partials
// first, the level-1 sums after them.
static hipError_t reduce_launches(int T, int E, int K, int nblk, float* part, const int32_t* counts,
                                  float* z_loss, float* aux_topk, hipStream_t s) {
    const int G = nblk < RL_G ? nblk : RL_G;
    double* lvl1 = reinterpret_cast<double*>(reinterpret_cast<char*>(part) +
                                             align_up((size_t)nblk * (E + 1) * sizeof(float), 256));
    router_losses_reduce1_kernel<<<G, 256, 0, s>>>(E, nblk, G, part, lvl1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    router_losses_reduce2_kernel<<<1, 1024, 0, s>>>(T, E, K, G, lvl1, counts, z_loss, aux_topk);
    return hipGetLastError();
}

hipError_t launch_router_losses_reduce(int T, int E, int K, int nblk, float* part, const int32_t* counts,
                                       float* z_loss, float* aux_topk, hipStream_t s) {
    hipError_t err = hipSuccess;
    MOE_TIMED_LAUNCH(MOE_KERNEL_ROUTER_LOSSES, s, err = reduce_launches(T, E, K, nblk, part, counts, z_loss, aux_topk, s));
    return err;
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
    return reduce_launches(T, E, K, nblk, part, counts, z_loss, aux_topk, s);
}

}  // namespace moe
