// Router: scores x W_r, per-expert bias, softmax over all experts, top-K with
// the lower expert index first on ties, and renormalisation over the K chosen.
// MoE notes (www.cf-1.com/news/5905749) §1.2 and §2 steps 1-3; MoE inference
// engineering page (ybb.press/quantum-computing/18594) §1 and §1.2.
//
// bf16 path: one fused kernel.  A workgroup owns 32 tokens; W_r is staged
// through LDS in 64-row slices, transposed to [expert][k] so that each MFMA
// operand is one 16-byte LDS read; x is read straight from HBM with 16-byte
// loads.  The 32 x E logit tile then stays in LDS for the routing phase, where
// each wave routes one token at a time (lanes own experts lane, lane+64, ...).
// fp32 path: a plain FMA kernel for the scores, then the same routing phase.
#include <math.h>

#include "../device_common.h"
#include "../launch.h"

namespace moe {

constexpr int RT_BT = 32;            // tokens per workgroup
constexpr int RT_KC = 64;            // rows of W_r staged per step
constexpr int RT_LDSK = RT_KC + 8;   // padded LDS row of the transposed W_r slice (bf16)
constexpr int RT_THREADS = 256;

// Route one token whose E logits are `lg`; the wave computes it together.
// psum[j] accumulates this wave's probabilities of expert lane + 64 j.
template <int MAXV>
__device__ __forceinline__ void route_token(const float* lg, int E, int K, const float* bias,
                                            float* probs_row, int32_t* ids_row, float* w_row,
                                            float (&psum)[MAXV]) {
    const int lane = lane_id();
    float v[MAXV];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
        const int e = lane + j * kWave;
        if (e < E) {
            const float b = bias ? bias[e] : 0.0f;
            v[j] = lg[e] + b;  // one fp32 addition, round to nearest even
            m = fmaxf(m, v[j]);
        } else {
            v[j] = -INFINITY;
        }
    }
    m = wave_max(m);
    float s = 0.0f;
    float ex[MAXV];
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
        const int e = lane + j * kWave;
        ex[j] = (e < E) ? expf(v[j] - m) : 0.0f;
        s += ex[j];
    }
    s = wave_sum(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
        const int e = lane + j * kWave;
        if (e < E) {
            const float p = ex[j] * inv;
            psum[j] += p;
            if (probs_row) probs_row[e] = p;
        }
    }
    // Top-K: K rounds of a wave-wide arg-max over the experts not yet taken.
    // Order: larger value first; equal values (including -0 vs +0, which
    // compare equal) go to the lower expert index.
    uint32_t taken = 0u;
    float my_e = 0.0f;
    int my_id = 0;
    float sel_sum = 0.0f;
    for (int k = 0; k < K; ++k) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < MAXV; ++j) {
            const int e = lane + j * kWave;
            if (e < E && !((taken >> j) & 1u)) {
                if (v[j] > bv || (v[j] == bv && e < bi)) {
                    bv = v[j];
                    bi = e;
                }
            }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float ov = __shfl_xor(bv, o);
            const int oi = __shfl_xor(bi, o);
            if (ov > bv || (ov == bv && oi < bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
        const float ek = expf(bv - m);  // same value as ex[] of the winner
        sel_sum += ek;
        if (lane == k) {
            my_e = ek;
            my_id = bi;
        }
    }
    if (lane < K) {
        ids_row[lane] = my_id;
        w_row[lane] = my_e / sel_sum;
    }
}

// Routing phase shared by the kernels: tokens t0 .. t0+RT_BT-1, logits of
// token t at lg + (t - t0) * lg_stride.  Writes the per-block prob sums.
template <int MAXV>
__device__ void route_block(int T, int E, int K, int t0, const float* lg, int lg_stride,
                            const float* bias, float* probs, int32_t* ids, float* w,
                            float* psum_part, float* red /* LDS, 4*E floats */) {
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    float psum[MAXV];
#pragma unroll
    for (int j = 0; j < MAXV; ++j) psum[j] = 0.0f;
    for (int tt = wave; tt < RT_BT; tt += RT_THREADS / kWave) {
        const int t = t0 + tt;
        if (t >= T) break;
        route_token<MAXV>(lg + (size_t)tt * lg_stride, E, K, bias,
                          probs ? probs + (size_t)t * E : nullptr, ids + (size_t)t * K,
                          w + (size_t)t * K, psum);
    }
    if (psum_part) {
        __syncthreads();  // red may alias the logit tile
#pragma unroll
        for (int j = 0; j < MAXV; ++j) {
            const int e = lane + j * kWave;
            if (e < E) red[wave * E + e] = psum[j];
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += RT_THREADS) {
            float acc = red[e];
            for (int wv = 1; wv < RT_THREADS / kWave; ++wv) acc += red[wv * E + e];
            psum_part[(size_t)blockIdx.x * E + e] = acc;
        }
    }
}

template <int MAXV>
__global__ __launch_bounds__(RT_THREADS) void router_bf16_kernel(
    int T, int d, int E, int K, int ep_max, const bf16* __restrict__ x,
    const bf16* __restrict__ wr, const float* __restrict__ bias, float* __restrict__ logits,
    float* __restrict__ probs, float* __restrict__ psum_part, int32_t* __restrict__ ids,
    float* __restrict__ w) {
    extern __shared__ __align__(16) char smem[];
    float* lg = reinterpret_cast<float*>(smem);                                  // [RT_BT][E]
    bf16* wt = reinterpret_cast<bf16*>(smem + ((RT_BT * E * 4 + 15) & ~15));  // [ep_max][RT_LDSK]
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int t0 = blockIdx.x * RT_BT;
    const int mb = wave & 1;      // 16-token block of this wave
    const int npar = wave >> 1;   // this wave takes expert blocks npar, npar + 2, ...
    const int tok = min(t0 + mb * 16 + (lane & 15), T - 1);
    const bf16* xrow = x + (size_t)tok * d;
    const int kq = (lane >> 4) * 8;
    const bool vec_ok = (E % 8) == 0;

    for (int e0 = 0; e0 < E; e0 += ep_max) {
        const int ep = min(ep_max, E - e0);
        const int nblk = (ep + 15) / 16;
        f32x4 acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int k0 = 0; k0 < d; k0 += RT_KC) {
            __syncthreads();
            // Stage W_r[k0 .. k0+RT_KC) x [e0 .. e0+ep) as wt[e][k].
            if (vec_ok) {
                const int nv = RT_KC * (ep / 8);
                for (int v = tid; v < nv; v += RT_THREADS) {
                    const int kk = v / (ep / 8);
                    const int ee = (v - kk * (ep / 8)) * 8;
                    u32x4 val = load16_or_zero(wr + (size_t)(k0 + kk) * E + e0 + ee, k0 + kk < d);
                    const bf16x8 b = as_bf16x8(val);
#pragma unroll
                    for (int i = 0; i < 8; ++i) wt[(ee + i) * RT_LDSK + kk] = b[i];
                }
            } else {
                const int ne = RT_KC * ep;
                for (int v = tid; v < ne; v += RT_THREADS) {
                    const int kk = v / ep;
                    const int ee = v - kk * ep;
                    wt[ee * RT_LDSK + kk] = (k0 + kk < d) ? wr[(size_t)(k0 + kk) * E + e0 + ee] : (bf16)0.0f;
                }
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < RT_KC; ks += 32) {
                const int k = k0 + ks + kq;
                const bf16x8 a = as_bf16x8(load16_or_zero(xrow + k, k < d));
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int nb = npar + 2 * j;
                    if (nb < nblk) {
                        int er = nb * 16 + (lane & 15);
                        er = er < ep ? er : ep - 1;
                        const bf16x8 b = *reinterpret_cast<const bf16x8*>(&wt[er * RT_LDSK + ks + kq]);
                        acc[j] = mfma16(a, b, acc[j]);
                    }
                }
            }
        }
        // acc[j][i] = logit of token (lane/16)*4 + i of this wave's block, expert nb*16 + lane%16
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int nb = npar + 2 * j;
            if (nb < nblk) {
                const int e = e0 + nb * 16 + (lane & 15);
                if (e < e0 + ep) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int tt = mb * 16 + (lane >> 4) * 4 + i;
                        const int t = t0 + tt;
                        lg[tt * E + e] = acc[j][i];
                        if (t < T) logits[(size_t)t * E + e] = acc[j][i];
                    }
                }
            }
        }
    }
    __syncthreads();
    // psum reduction reuses the W_r staging area (4 * E floats fit in it).
    route_block<MAXV>(T, E, K, t0, lg, E, bias, probs, ids, w, psum_part,
                      reinterpret_cast<float*>(wt));
}

// Routing of given fp32 logits (no GEMM): the x == NULL mode and the fp32 path.
template <int MAXV>
__global__ __launch_bounds__(RT_THREADS) void route_logits_kernel(
    int T, int E, int K, const float* __restrict__ logits, const float* __restrict__ bias,
    float* __restrict__ probs, float* __restrict__ psum_part, int32_t* __restrict__ ids,
    float* __restrict__ w) {
    extern __shared__ __align__(16) char smem[];
    const int t0 = blockIdx.x * RT_BT;
    route_block<MAXV>(T, E, K, t0, logits + (size_t)t0 * E, E, bias, probs, ids, w, psum_part,
                      reinterpret_cast<float*>(smem));
}

// fp32 scores: one thread per (token, expert), plain FMA over d.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(int T, int d, int E,
                                                               const float* __restrict__ x,
                                                               const float* __restrict__ wr,
                                                               float* __restrict__ logits) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)T * E) return;
    const int t = (int)(i / E);
    const int e = (int)(i - (size_t)t * E);
    const float* xr = x + (size_t)t * d;
    float s = 0.0f;
    for (int j = 0; j < d; ++j) s = fmaf(xr[j], wr[(size_t)j * E + e], s);
    logits[i] = s;
}

// prob_sum[e] = sum over blocks (ascending) of the per-block sums, in double.
__global__ __launch_bounds__(256) void psum_reduce_kernel(int nblk, int E,
                                                         const float* __restrict__ part,
                                                         float* __restrict__ prob_sum) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    double s = 0.0;
    for (int b = 0; b < nblk; ++b) s += (double)part[(size_t)b * E + e];
    prob_sum[e] = (float)s;
}

int router_num_blocks(int T, int /*dtype*/) { return (T + RT_BT - 1) / RT_BT; }

size_t router_ws_bytes(int T, int E, int dtype) {
    return align_up((size_t)router_num_blocks(T, dtype) * E * sizeof(float), 256);
}

static int route_ep_max(int E) { return E > 512 ? 128 : 256; }

static size_t router_lds_bytes(int E) {
    const size_t lg = (RT_BT * (size_t)E * 4 + 15) / 16 * 16;
    size_t wt = (size_t)route_ep_max(E) * RT_LDSK * 2;
    const size_t red = (size_t)4 * E * 4;
    if (wt < red) wt = red;
    return lg + wt;
}

template <int MAXV>
static hipError_t launch_router_t(int T, int d, int E, int K, int dtype, const void* x,
                                  const void* wr, const float* bias, float* logits, float* probs,
                                  float* psum_part, int32_t* ids, float* w, hipStream_t s) {
    const int nblk = router_num_blocks(T, dtype);
    if (x != nullptr && dtype == MOE_DTYPE_BF16) {
        const size_t lds = router_lds_bytes(E);
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t err = hipFuncSetAttribute((const void*)router_bf16_kernel<MAXV>,
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 160 * 1024);
            if (err != hipSuccess) return err;
            attr_set = true;
        }
        MOE_TIMED_LAUNCH(MOE_KERNEL_ROUTER, s,
                         router_bf16_kernel<MAXV><<<nblk, RT_THREADS, lds, s>>>(
                             T, d, E, K, route_ep_max(E), (const bf16*)x, (const bf16*)wr, bias,
                             logits, probs, psum_part, ids, w));
        return hipGetLastError();
    }
    if (x != nullptr) {  // fp32 scores first
        const size_t n = (size_t)T * E;
        router_logits_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
            T, d, E, (const float*)x, (const float*)wr, logits);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    MOE_TIMED_LAUNCH(MOE_KERNEL_ROUTER, s,
                     route_logits_kernel<MAXV><<<nblk, RT_THREADS, (size_t)4 * E * 4, s>>>(
                         T, E, K, logits, bias, probs, psum_part, ids, w));
    return hipGetLastError();
}

hipError_t launch_router(int T, int d, int E, int K, int dtype, const void* x,
                         const void* w_router, const float* bias, float* logits, float* probs,
                         float* prob_sum, int32_t* ids, float* w, void* ws, hipStream_t s) {
    float* part = prob_sum ? reinterpret_cast<float*>(ws) : nullptr;
    hipError_t err;
    if (E <= 64)
        err = launch_router_t<1>(T, d, E, K, dtype, x, w_router, bias, logits, probs, part, ids, w, s);
    else if (E <= 256)
        err = launch_router_t<4>(T, d, E, K, dtype, x, w_router, bias, logits, probs, part, ids, w, s);
    else
        err = launch_router_t<16>(T, d, E, K, dtype, x, w_router, bias, logits, probs, part, ids, w, s);
    if (err != hipSuccess || !prob_sum) return err;
    psum_reduce_kernel<<<(E + 255) / 256, 256, 0, s>>>(router_num_blocks(T, dtype), E, part, prob_sum);
    return hipGetLastError();
}

}  // namespace moe
