// Router: scores x W_r, per-expert bias, softmax over all experts, top-K with
// the lower expert index first on ties, and renormalisation over the K chosen.
// MoE notes (www.cf-1.com/news/5905749) §1.2 and §2 steps 1-3; MoE inference
// engineering page (ybb.press/quantum-computing/18594) §1 and §1.2.
//
// bf16 path, three kernels:
//   transpose : W_r [d, E] -> W_r^T [E, d] in the workspace, so that both MFMA
//               operands are contiguous along d;
//   gemm      : logits as a batched matmul over all tokens (§2.1 of the notes):
//               each wave owns 16 tokens x 16*NEB experts over one slice of d
//               and streams its token rows from HBM with 16x16x32 bf16 MFMAs
//               (two 128-wide chunks of x in flight while the current one is
//               multiplied; the workgroup's W_r^T rows arrive in LDS by DMA
//               from L2).  Small token counts split d over the grid so that
//               enough waves stream x; the per-slice partial scores go to the
//               workspace;
//   route     : a wave takes one or two tokens, sums their slices in slice
//               order (a fixed order, so the logits are deterministic), adds
//               the bias, and runs the softmax, the top-K and the
//               renormalisation with lanes owning experts lane, lane + 64, ...
// fp32 path: a plain FMA kernel for the scores, then the same route kernel.
#include <math.h>

#include "../device_common.h"
#include "../launch.h"
#include "dispatch_small.h"

namespace moe {

constexpr int RT_THREADS = 256;
// Tokens per route wave, by scores per lane (MAXV).  With at most 64 experts a
// token's routing is short, so a wave takes two tokens and has the score
// loads of both in flight at once.  With more experts each token runs K
// arg-max rounds over several scores per lane, a chain of cross-lane
// shuffles; one token per wave then leaves four waves per SIMD to hide that
// latency.  (Measured on the route kernel alone: 15.5 us at T = 8192, E = 8
// and 15.4 us at T = 16384, E = 64 with two tokens per wave, against 22.0 and
// 18.5 us with four; 19.5 us at T = 4096, E = 256, K = 8 with one, against
// 26.4 with two and 42.4 with four.)
__host__ __device__ constexpr int rt_tpw(int maxv) { return maxv == 1 ? 2 : 1; }
static int router_maxv(int E) { return E <= 64 ? 1 : (E <= 256 ? 4 : 16); }
constexpr int RG_KCH = 128;  // d chunk per gemm iteration

// ---- route ---------------------------------------------------------------------
// Route one token whose scores this lane holds for experts lane + 64 j.  The
// wave computes it together.  psum[j] accumulates this wave's probabilities of
// expert lane + 64 j.  flags: MOE_FLAG_BIAS_SELECT_ONLY (the bias steers the
// choice only; probabilities and weights come from the unbiased scores),
// MOE_FLAG_COMBINE_MEAN (every weight is 1/K).
//
// With `losses`, the router regularisers of the MoE notes §3.2 are gathered
// from the same max and sum of exponentials: zacc (wave-uniform) adds the
// token's squared log-sum-exp of the unbiased scores, and csum[j] adds the
// routing probability (softmax of scores + bias over all experts) of expert
// lane + 64 j when the token chose it.
template <int MAXV>
__device__ __forceinline__ void route_token(const float (&lg)[MAXV], int E, int K, const float* bias,
                                            int flags, float* probs_row, int32_t* ids_row,
                                            float* w_row, float (&psum)[MAXV], bool losses = false,
                                            float* zacc = nullptr, float* csum = nullptr) {
    const int lane = lane_id();
    const bool sel_only = (flags & MOE_FLAG_BIAS_SELECT_ONLY) != 0;
    float v[MAXV];  // selection keys: scores + bias
    float u[MAXV];  // softmax inputs: the same, or the unbiased scores
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
        const int e = lane + j * kWave;
        if (e < E) {
            const float b = bias ? bias[e] : 0.0f;
            v[j] = lg[j] + b;  // one fp32 addition, round to nearest even
            u[j] = sel_only ? lg[j] : v[j];
            m = fmaxf(m, u[j]);
        } else {
            v[j] = -INFINITY;
            u[j] = -INFINITY;
        }
    }
    m = wave_max(m);
    float s = 0.0f;
    float ex[MAXV];
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
        const int e = lane + j * kWave;
        ex[j] = (e < E) ? expf(u[j] - m) : 0.0f;
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
    // Regularisers: the unbiased log-sum-exp is the softmax's own when the
    // softmax ran on the unbiased scores, and the routing probabilities are
    // the softmax's own when it ran on the biased ones.
    float mb = m, sb = s;
    if (losses) {
        float m0 = m, s0 = s;
        if (bias && !sel_only) {
            m0 = -INFINITY;
#pragma unroll
            for (int j = 0; j < MAXV; ++j)
                if (lane + j * kWave < E) m0 = fmaxf(m0, lg[j]);
            m0 = wave_max(m0);
            s0 = 0.0f;
#pragma unroll
            for (int j = 0; j < MAXV; ++j)
                if (lane + j * kWave < E) s0 += expf(lg[j] - m0);
            s0 = wave_sum(s0);
        }
        if (bias && sel_only) {
            mb = -INFINITY;
#pragma unroll
            for (int j = 0; j < MAXV; ++j)
                if (lane + j * kWave < E) mb = fmaxf(mb, v[j]);
            mb = wave_max(mb);
            sb = 0.0f;
#pragma unroll
            for (int j = 0; j < MAXV; ++j)
                if (lane + j * kWave < E) sb += expf(v[j] - mb);
            sb = wave_sum(sb);
        }
        const float lse = m0 + logf(s0);
        *zacc += lse * lse;
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
        if ((bi & (kWave - 1)) == lane) {
            taken |= 1u << (bi / kWave);
            if (losses) {
                const float pc = expf(bv - mb) / sb;  // routing probability of the winner
#pragma unroll
                for (int j = 0; j < MAXV; ++j)
                    if (j == bi / kWave) csum[j] += pc;
            }
        }
        float uw = bv;  // softmax input of the winner
        if (sel_only) {
            float mine = 0.0f;
#pragma unroll
            for (int j = 0; j < MAXV; ++j)
                if (j == bi / kWave) mine = u[j];
            uw = __shfl(mine, bi & (kWave - 1));
        }
        const float ek = expf(uw - m);  // same value as ex[] of the winner
        sel_sum += ek;
        if (lane == k) {
            my_e = ek;
            my_id = bi;
        }
    }
    if (lane < K) {
        ids_row[lane] = my_id;
        w_row[lane] = (flags & MOE_FLAG_COMBINE_MEAN) ? 1.0f / (float)K : my_e / sel_sum;
    }
}

// src holds nsplit slices [nsplit][T][E] of partial scores (nsplit = 1: the
// scores themselves).  When logits_out is given, the summed scores are written
// there.  psum_part (optional) receives this block's per-expert probability sums.
// loss_part (optional): this block's router-regulariser partials, the
// chosen-probability sums at [blockIdx.x][E] and the sum of squared
// log-sum-exps at [gridDim.x * E + blockIdx.x] (router_losses_reduce_kernel
// adds them up).
template <int MAXV>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(
    int T, int E, int K, int flags, int nsplit, const float* __restrict__ src,
    float* __restrict__ logits_out, const float* __restrict__ bias, float* __restrict__ probs,
    float* __restrict__ psum_part, float* __restrict__ loss_part,
    int32_t* __restrict__ ids, float* __restrict__ w) {
    extern __shared__ float red[];  // [RT_THREADS / kWave][E], then [RT_THREADS / kWave] z sums
    const int wave = threadIdx.x / kWave;
    const int lane = lane_id();
    const bool losses = loss_part != nullptr;
    float psum[MAXV], csum[MAXV];
    float zacc = 0.0f;
#pragma unroll
    for (int j = 0; j < MAXV; ++j) psum[j] = csum[j] = 0.0f;
    // Wave w routes tokens blockIdx.x * BT + w * TPW + [0, TPW): the scores
    // of all of them are loaded first (every load in flight at once), then
    // the tokens are routed in order.
    constexpr int RT_TPW = rt_tpw(MAXV);
    constexpr int BT = RT_TPW * RT_THREADS / kWave;
    const size_t slice = (size_t)T * E;
    const int t0 = blockIdx.x * BT + wave * RT_TPW;
    float lgs[RT_TPW][MAXV];
#pragma unroll
    for (int i = 0; i < RT_TPW; ++i) {
        const int t = min(t0 + i, T - 1);
#pragma unroll
        for (int j = 0; j < MAXV; ++j) {
            const int e = lane + j * kWave;
            lgs[i][j] = e < E ? src[(size_t)t * E + e] : 0.0f;
        }
    }
    // further slices of the scores, added in slice order
    for (int sp = 1; sp < nsplit; ++sp) {
        float v[RT_TPW][MAXV];
#pragma unroll
        for (int i = 0; i < RT_TPW; ++i) {
            const int t = min(t0 + i, T - 1);
#pragma unroll
            for (int j = 0; j < MAXV; ++j) {
                const int e = lane + j * kWave;
                v[i][j] = e < E ? src[(size_t)sp * slice + (size_t)t * E + e] : 0.0f;
            }
        }
#pragma unroll
        for (int i = 0; i < RT_TPW; ++i)
#pragma unroll
            for (int j = 0; j < MAXV; ++j) lgs[i][j] += v[i][j];
    }
#pragma unroll
    for (int i = 0; i < RT_TPW; ++i) {
        const int t = t0 + i;
        if (t >= T) break;
        if (logits_out) {
#pragma unroll
            for (int j = 0; j < MAXV; ++j) {
                const int e = lane + j * kWave;
                if (e < E) logits_out[(size_t)t * E + e] = lgs[i][j];
            }
        }
        route_token<MAXV>(lgs[i], E, K, bias, flags, probs ? probs + (size_t)t * E : nullptr,
                          ids + (size_t)t * K, w + (size_t)t * K, psum, losses, &zacc, csum);
    }
    // Per-block sums over the waves, in wave order (a fixed order).
    auto block_sums = [&](const float (&acc)[MAXV], float* out) {
#pragma unroll
        for (int j = 0; j < MAXV; ++j) {
            const int e = lane + j * kWave;
            if (e < E) red[wave * E + e] = acc[j];
        }
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += RT_THREADS) {
            float a = red[e];
            for (int wv = 1; wv < RT_THREADS / kWave; ++wv) a += red[wv * E + e];
            out[(size_t)blockIdx.x * E + e] = a;
        }
        __syncthreads();
    };
    if (psum_part) block_sums(psum, psum_part);
    if (losses) {
        float* zred = red + (RT_THREADS / kWave) * E;
        if (lane == 0) zred[wave] = zacc;
        block_sums(csum, loss_part);
        if (threadIdx.x == 0) {
            float a = zred[0];
            for (int wv = 1; wv < RT_THREADS / kWave; ++wv) a += zred[wv];
            loss_part[(size_t)gridDim.x * E + blockIdx.x] = a;
        }
    }
}

// prob_sum[e] = sum over route blocks of the per-block sums: one workgroup
// per expert; thread i adds blocks i, i + 256, ... in block order in double
// (eight loads in flight), then a fixed pairwise tree over the 256 threads.
__global__ __launch_bounds__(256) void psum_reduce_kernel(int nblk, int E,
                                                         const float* __restrict__ part,
                                                         float* __restrict__ prob_sum) {
    __shared__ double red[256];
    const int e = blockIdx.x;
    double s = 0.0;
    for (int b0 = threadIdx.x; b0 < nblk; b0 += 8 * 256) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = b0 + q * 256 < nblk ? part[(size_t)(b0 + q * 256) * E + e] : 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) s += (double)v[q];
    }
    red[threadIdx.x] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
        __syncthreads();
    }
    if (threadIdx.x == 0) prob_sum[e] = (float)red[0];
}

// ---- scores ---------------------------------------------------------------------
// W_r [d, E] -> W_r^T [E, d] through a padded LDS tile.
__global__ __launch_bounds__(256) void router_transpose_kernel(int d, int E, const bf16* __restrict__ wr,
                                                              bf16* __restrict__ wrt) {
    __shared__ bf16 tile[64][65];
    const int k0 = blockIdx.x * 64;
    const int e0 = blockIdx.y * 64;
    bf16 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {  // all sixteen loads in flight together
        const int i = threadIdx.x + q * 256;
        const int kk = i / 64, ee = i % 64;
        v[q] = (k0 + kk < d && e0 + ee < E) ? wr[(size_t)(k0 + kk) * E + e0 + ee] : (bf16)0.0f;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int i = threadIdx.x + q * 256;
        tile[i / 64][i % 64] = v[q];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
        const int ee = i / 64, kk = i % 64;
        if (k0 + kk < d && e0 + ee < E) wrt[(size_t)(e0 + ee) * d + k0 + kk] = tile[kk][ee];
    }
}

// out[split][t][e] = sum over d in this split's slice of x[t][k] * W_r^T[e][k].
// Workgroup tile: 64 tokens (16 per wave) x 16*NEB experts.  The W_r^T rows
// of each 128-wide chunk of d are shared by the four waves through LDS: they
// arrive by DMA (global_load_lds) into a ring of three buffers, with chunk c
// of row r in slot c ^ (r % 16) so that the fragment reads of 16 consecutive
// rows fall in distinct banks.  Token rows come straight from HBM into a ring
// of three register sets.  Both streams run two chunks ahead of the MFMAs
// (the kernel is bound by memory latency: little arithmetic per byte).
// Every chunk issues the same loads (the ones past the slice at clamped
// addresses, their values discarded), so one wait count fits every step.
// Lane (r = lane % 16, g = lane / 16); in each 32-wide step both operands
// take k = 32 s + 8 g + [0, 8).
template <int NEB>
__global__ __launch_bounds__(256) void router_gemm_kernel(int T, int d, int E, int kspan,
                                                         const bf16* __restrict__ x,
                                                         const bf16* __restrict__ wrt,
                                                         float* __restrict__ out) {
    constexpr int ROWS = 16 * NEB;                // W_r^T rows per workgroup
    constexpr int CH = ROWS * RG_KCH;             // bf16 elements of one chunk
    constexpr int NLD = ROWS * RG_KCH * 2 / 16 / 256;  // 16-byte DMA loads per thread per chunk
    constexpr int NX = 4;                         // 16-byte token loads per thread per chunk
    static_assert(NLD >= 1, "chunk covers the workgroup");
    __shared__ __align__(1024) bf16 wb0[CH], wb1[CH], wb2[CH];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int lane = lane_id();
    const int rl = lane & 15;
    const int g = lane >> 4;
    const int tb = blockIdx.x * 4 + wave;
    const bool active = tb * 16 < T;  // idle waves still take part in the loads and barriers
    const int eb0 = blockIdx.y * ROWS;
    const int k_beg = blockIdx.z * kspan;
    const int k_end = min(d, k_beg + kspan);
    const int nch = max(0, (k_end - k_beg + RG_KCH - 1) / RG_KCH);
    // DMA: thread p fills LDS slots p + 256 i (16 bytes each) = row (p + 256 i) / 16,
    // slot (p + 256 i) % 16, holding chunk slot ^ (row % 16) of that row.
    const bf16* wsrc[NLD];
    int wcol[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int q = (int)threadIdx.x + 256 * i;
        const int row = q / 16;
        wcol[i] = ((q % 16) ^ (row & 15)) * 8;
        wsrc[i] = wrt + (size_t)min(eb0 + row, E - 1) * d;
    }
    auto issue = [&](int c, bf16* dst) __attribute__((always_inline)) {
        const int kc = k_beg + min(c, max(nch - 1, 0)) * RG_KCH;
#pragma unroll
        for (int i = 0; i < NLD; ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(wsrc[i] + min(kc + wcol[i], d - 8)),
                (__attribute__((address_space(3))) void*)(dst + (size_t)(wave * kWave + 256 * i) * 8), 16, 0, 0);
    };
    const int kl = g * 8;
    const bf16* xrow = x + (size_t)min(tb * 16 + rl, T - 1) * d;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // raw loads; the values past the slice (or of an idle wave) are zeroed at
    // their use, so that nothing waits for a load before then
    auto load_x = [&](int c, u32x4 (&xv)[NX]) __attribute__((always_inline)) {
#pragma unroll
        for (int s = 0; s < NX; ++s) xv[s] = load16(xrow + min(k_beg + c * RG_KCH + s * 32 + kl, d - 8));
    };
    f32x4 acc[NEB];
#pragma unroll
    for (int j = 0; j < NEB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // chunk c of the slice: wait for its W_r^T DMA and token loads (only chunk
    // c + 1's may still be in flight), make the DMA visible to every wave,
    // refill the ring slot of chunk c - 1 with chunk c + 2, then multiply.
    auto step = [&](int c, const bf16* cur, bf16* nxt2, const u32x4 (&xc)[NX], u32x4 (&xn2)[NX])
        __attribute__((always_inline)) {
        // (a plain barrier: a fence here would wait for every load in flight;
        // the ring slot refilled below was last read by the MFMAs of chunk
        // c - 1, whose fragment reads have completed)
        __builtin_amdgcn_s_waitcnt(((NLD + NX) & 15) | (7 << 4) | (15 << 8) | ((((NLD + NX) >> 4) & 3) << 14));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(c + 2, nxt2);
        load_x(c + 2, xn2);
        // W_r^T fragments of step s + 1 are read while step s is multiplied
        bf16x8 wv[2][NEB];
        auto rd = [&](int s, bf16x8 (&f)[NEB]) {
            const int slot = ((4 * s + g) ^ rl) * 8;
#pragma unroll
            for (int j = 0; j < NEB; ++j)
                f[j] = *reinterpret_cast<const bf16x8*>(cur + (j * 16 + rl) * RG_KCH + slot);
        };
        rd(0, wv[0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3) rd(s + 1, wv[(s + 1) & 1]);
            const bool ok = active && k_beg + c * RG_KCH + s * 32 + kl < k_end;
            const u32x4 xs = ok ? xc[s] : zero;
#pragma unroll
            for (int j = 0; j < NEB; ++j) acc[j] = mfma16(as_bf16x8(xs), wv[s & 1][j], acc[j]);
        }
    };
    u32x4 xa[NX], xb[NX], xc[NX];
    issue(0, wb0);
    load_x(0, xa);
    issue(1, wb1);
    load_x(1, xb);
    const int nch3 = nch - nch % 3;
    for (int c = 0; c < nch3; c += 3) {
        step(c, wb0, wb2, xa, xc);
        step(c + 1, wb1, wb0, xb, xa);
        step(c + 2, wb2, wb1, xc, xb);
    }
    // the last nch % 3 chunks start again at ring slot 0
    if (nch3 < nch) step(nch3, wb0, wb2, xa, xc);
    if (nch3 + 1 < nch) step(nch3 + 1, wb1, wb0, xb, xa);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no DMA may outlive the workgroup
    if (!active) return;
    // acc[j][i]: token tb*16 + 4g + i, expert eb0 + 16 j + rl
    float* o = out + (size_t)blockIdx.z * T * E;
#pragma unroll
    for (int j = 0; j < NEB; ++j) {
        const int e = eb0 + j * 16 + rl;
        if (e >= E) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tb * 16 + g * 4 + i;
            if (t < T) o[(size_t)t * E + e] = acc[j][i];
        }
    }
}

// fp32 scores: one wave per (token, expert); lane l takes j = l, l + 64, ...
// of the token row, then a fixed-order wave sum.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(int T, int d, int E,
                                                               const float* __restrict__ x,
                                                               const float* __restrict__ wr,
                                                               float* __restrict__ logits) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) / kWave;
    const int lane = lane_id();
    if (i >= (size_t)T * E) return;
    const int t = (int)(i / E);
    const int e = (int)(i - (size_t)t * E);
    const float* xr = x + (size_t)t * d;
    float s = 0.0f;
    for (int j = lane; j < d; j += kWave) s = fmaf(xr[j], wr[(size_t)j * E + e], s);
    s = wave_sum(s);
    if (lane == 0) logits[i] = s;
}

// ---- small batches: two launches for the whole front of the layer -----------
// For decode-sized batches (T <= 64 tokens, E <= 16 experts):
//   small_gemm : RS_SLICES workgroups, one slice of d each; the workgroup
//                copies its rows of W_r (one contiguous block of [d, E]) into
//                LDS, its four waves take a quarter of the slice each and run
//                16x16x32 MFMAs of the token rows (read straight from HBM)
//                against W_r^T fragments gathered from LDS, and the four
//                quarters are added in order into the slice's partial scores;
//   route_dispatch_small : one workgroup of 1024 threads adds the slices in
//                slice order, routes one token per wave (route_token above)
//                and dispatches the T*K assignments (dispatch_small_block).
// Same arithmetic as the general kernels except the slicing of d, which only
// changes fp32 rounding.
constexpr int RS_SLICES = 16;
constexpr int RS_MAXT = 64;
constexpr int RS_MAXE = 16;
constexpr int RS_WLDS = 8192;  // W_r elements staged per workgroup

__host__ __device__ static inline int rs_kslice(int d) { return ((d + RS_SLICES - 1) / RS_SLICES + 127) / 128 * 128; }

bool route_dispatch_small_ok(int T, int d, int E, int K, int dtype) {
    return dtype == MOE_DTYPE_BF16 && T >= 1 && T <= RS_MAXT && E <= RS_MAXE && K <= E && d % 8 == 0 &&
           rs_kslice(d) * E <= RS_WLDS;
}

size_t route_dispatch_small_ws_bytes(int T, int E) { return align_up((size_t)RS_SLICES * T * E * sizeof(float), 256); }

template <int NTB>
__global__ __launch_bounds__(256) void small_gemm_kernel(int T, int d, int E, const bf16* __restrict__ x,
                                                         const bf16* __restrict__ wr, float* __restrict__ part) {
    __shared__ __align__(16) bf16 wflat[RS_WLDS];
    __shared__ float red[4][RS_MAXT * RS_MAXE];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int lane = lane_id();
    const int rl = lane & 15;
    const int g = lane >> 4;
    const int ks = rs_kslice(d);
    const int kb = blockIdx.x * ks;
    // rows [kb, kb + ks) of W_r are bytes [2 E kb, 2 E (kb + ks)) of it
    {
        const char* src = reinterpret_cast<const char*>(wr) + (size_t)kb * E * 2;
        const long valid = max(0L, ((long)d - kb) * E * 2);
        char* dst = reinterpret_cast<char*>(wflat);
        for (int off = threadIdx.x * 16; off < ks * E * 2; off += 256 * 16)
            store16(dst + off, load16_or_zero(src + off, off < valid));
    }
    // this wave: k in [kb + wave * ks / 4, + ks / 4), in steps of 32
    const int q = ks / 4;
    const int kq = kb + wave * q;
    u32x4 xf[NTB][4];
    f32x4 acc[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < q / 32; s0 += 4) {
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = kq + (s0 + j) * 32 + g * 8;
                const int t = min(tb * 16 + rl, T - 1);
                xf[tb][j] = load16_or_zero(x + (size_t)t * d + k, s0 + j < q / 32 && k < d);
            }
        if (s0 == 0) __syncthreads();  // W_r rows staged
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (s0 + j < q / 32) {
                const int kl = wave * q + (s0 + j) * 32 + g * 8;  // local k of the fragment
                const bf16* wl = wflat + kl * E + min(rl, E - 1);
                bf16x8 wv;
#pragma unroll
                for (int i = 0; i < 8; ++i) wv[i] = wl[i * E];
                if (rl >= E) wv = bf16x8{};
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb) acc[tb] = mfma16(as_bf16x8(xf[tb][j]), wv, acc[tb]);
            }
        }
    }
    // acc[tb][i]: token tb*16 + 4g + i, expert rl
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tb * 16 + g * 4 + i;
            if (t < T && rl < E) red[wave][t * E + rl] = acc[tb][i];
        }
    __syncthreads();
    for (int i = threadIdx.x; i < T * E; i += 256)
        part[(size_t)blockIdx.x * T * E + i] = ((red[0][i] + red[1][i]) + red[2][i]) + red[3][i];
}

__global__ __launch_bounds__(1024) void route_dispatch_small_kernel(
    int T, int E, int K, int flags, int capacity, int nbits, const float* __restrict__ part,
    const float* __restrict__ bias, float* __restrict__ logits, float* __restrict__ probs,
    float* __restrict__ prob_sum, int32_t* __restrict__ ids, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
    int32_t* __restrict__ assign_row, int32_t* __restrict__ row_assign, float* __restrict__ z_loss,
    float* __restrict__ aux_topk) {
    __shared__ float lgs[RS_MAXT * RS_MAXE];
    __shared__ float pw[16][RS_MAXE];
    __shared__ float cw[16][RS_MAXE];
    __shared__ float zw[16];
    __shared__ double pe[RS_MAXE];
    __shared__ int sids[RS_MAXT * RS_MAXE];
    __shared__ int hist[1024];
    __shared__ int offs[1024];
    __shared__ int wave_tot[16];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int lane = lane_id();
    for (int i = threadIdx.x; i < T * E; i += 1024) {
        float v = part[i];
        for (int sl = 1; sl < RS_SLICES; ++sl) v += part[(size_t)sl * T * E + i];
        lgs[i] = v;
        if (logits) logits[i] = v;
    }
    __syncthreads();
    const bool losses = z_loss || aux_topk;
    float psum[1] = {0.0f}, csum[1] = {0.0f};
    float zacc = 0.0f;
    for (int t = wave; t < T; t += 16) {
        float lg[1] = {lane < E ? lgs[t * E + lane] : 0.0f};
        route_token<1>(lg, E, K, bias, flags, probs ? probs + (size_t)t * E : nullptr, sids + t * K,
                       w + (size_t)t * K, psum, losses, &zacc, csum);
    }
    if (lane < E) {
        pw[wave][lane] = psum[0];
        cw[wave][lane] = csum[0];
    }
    if (lane == 0) zw[wave] = zacc;
    __syncthreads();
    if (prob_sum && threadIdx.x < E) {
        double v = 0.0;
        for (int sl = 0; sl < 16; ++sl) v += (double)pw[sl][threadIdx.x];
        prob_sum[threadIdx.x] = (float)v;
    }
    for (int i = threadIdx.x; i < T * K; i += 1024) ids[i] = sids[i];
    const int cnt = dispatch_small_block(T * K, E, nbits, capacity, sids, counts, kept, offsets, assign_row,
                                         row_assign, hist, offs, wave_tot);
    if (losses) {
        // aux_topk = E sum_e f_e P'_e and z_loss = mean lse^2, in double, in
        // expert and wave order
        if ((int)threadIdx.x < E) {
            double ch = 0.0;
            for (int wv = 0; wv < 16; ++wv) ch += (double)cw[wv][threadIdx.x];
            pe[threadIdx.x] = (double)cnt / ((double)T * K) * (ch / (double)T);
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            if (aux_topk) {
                double a = 0.0;
                for (int e = 0; e < E; ++e) a += pe[e];
                *aux_topk = (float)((double)E * a);
            }
            if (z_loss) {
                double z = 0.0;
                for (int wv = 0; wv < 16; ++wv) z += (double)zw[wv];
                *z_loss = (float)(z / (double)T);
            }
        }
    }
}

hipError_t launch_route_dispatch_small(int T, int d, int E, int K, int flags, int capacity, const void* x,
                                       const void* w_router, const float* bias, float* logits,
                                       float* probs, float* prob_sum, int32_t* ids, float* w,
                                       int32_t* counts, int32_t* kept, int32_t* offsets,
                                       int32_t* assign_row, int32_t* row_assign, float* z_loss,
                                       float* aux_topk, void* ws, hipStream_t s) {
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    float* part = reinterpret_cast<float*>(ws);
    const int ntb = (T + 15) / 16;
    switch (ntb) {
        case 1: small_gemm_kernel<1><<<RS_SLICES, 256, 0, s>>>(T, d, E, (const bf16*)x, (const bf16*)w_router, part); break;
        case 2: small_gemm_kernel<2><<<RS_SLICES, 256, 0, s>>>(T, d, E, (const bf16*)x, (const bf16*)w_router, part); break;
        default: small_gemm_kernel<4><<<RS_SLICES, 256, 0, s>>>(T, d, E, (const bf16*)x, (const bf16*)w_router, part); break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    MOE_TIMED_LAUNCH(MOE_KERNEL_ROUTER, s,
                     route_dispatch_small_kernel<<<1, 1024, 0, s>>>(T, E, K, flags, capacity, nbits, part, bias,
                                                                    logits, probs, prob_sum, ids, w, counts,
                                                                    kept, offsets, assign_row, row_assign,
                                                                    z_loss, aux_topk));
    return hipGetLastError();
}

// ---- host side ------------------------------------------------------------------
static int router_neb(int E) {
    if (E <= 16) return 1;
    if (E <= 32) return 2;
    if (E <= 64) return 4;
    return 8;
}

// Slices of d for the score GEMM: enough waves to stream x, each slice a
// multiple of the chunk width, at most 8 slices and at most 8 MB of partial
// scores.
static int router_splits(int T, int d, int E) {
    const int neb = router_neb(E);
    const long waves = (long)((T + 15) / 16) * ((E + 16 * neb - 1) / (16 * neb));
    const int max_split = max(1, min(8, d / RG_KCH));  // the route kernel sums the slices in one batch
    int ns = 1;
    while (ns * 2 <= max_split && waves * ns < 4096 &&
           (size_t)(ns * 2) * T * E * sizeof(float) <= ((size_t)8 << 20))
        ns *= 2;
    return ns;
}

static int router_kspan(int d, int ns) {
    const int chunks = (d + RG_KCH - 1) / RG_KCH;
    return (chunks + ns - 1) / ns * RG_KCH;
}

int router_num_blocks(int T, int E) {
    const int bt = rt_tpw(router_maxv(E)) * RT_THREADS / kWave;
    return (T + bt - 1) / bt;
}

// Workspace: [W_r^T (bf16 with x)] [partial scores (bf16 with x, > 1 slice)] [prob-sum partials]
struct RouterLayout {
    size_t wrt, part, psum, total;
    int ns;
};

static RouterLayout router_layout(int T, int d, int E, int dtype) {
    RouterLayout L;
    size_t o = 0;
    L.ns = dtype == MOE_DTYPE_BF16 ? router_splits(T, d, E) : 1;
    L.wrt = o;
    if (dtype == MOE_DTYPE_BF16) o += align_up((size_t)E * d * 2, 256);
    L.part = o;
    if (L.ns > 1) o += align_up((size_t)L.ns * T * E * sizeof(float), 256);
    L.psum = o;
    o += align_up((size_t)router_num_blocks(T, E) * E * sizeof(float), 256);
    L.total = o;
    return L;
}

size_t router_ws_bytes(int T, int d, int E, int dtype) { return router_layout(T, d, E, dtype).total; }

template <int MAXV>
static hipError_t launch_route_t(int T, int E, int K, int flags, int nsplit, const float* src, float* logits_out,
                                 const float* bias, float* probs, float* psum_part, float* loss_part,
                                 int32_t* ids, float* w, hipStream_t s) {
    const int nblk = router_num_blocks(T, E);
    const size_t lds = ((size_t)(RT_THREADS / kWave) * E + RT_THREADS / kWave) * 4;
    MOE_TIMED_LAUNCH(MOE_KERNEL_ROUTER, s,
                     route_kernel<MAXV><<<nblk, RT_THREADS, lds, s>>>(
                         T, E, K, flags, nsplit, src, logits_out, bias, probs, psum_part, loss_part, ids, w));
    return hipGetLastError();
}

static hipError_t launch_route(int T, int E, int K, int flags, int nsplit, const float* src, float* logits_out,
                               const float* bias, float* probs, float* psum_part, float* loss_part,
                               int32_t* ids, float* w, hipStream_t s) {
    switch (router_maxv(E)) {
        case 1:
            return launch_route_t<1>(T, E, K, flags, nsplit, src, logits_out, bias, probs, psum_part, loss_part,
                                     ids, w, s);
        case 4:
            return launch_route_t<4>(T, E, K, flags, nsplit, src, logits_out, bias, probs, psum_part, loss_part,
                                     ids, w, s);
        default:
            return launch_route_t<16>(T, E, K, flags, nsplit, src, logits_out, bias, probs, psum_part, loss_part,
                                      ids, w, s);
    }
}

template <int NEB>
static void launch_gemm_t(int T, int d, int E, int ns, const bf16* x, const bf16* wrt, float* out,
                          hipStream_t s) {
    dim3 grid((unsigned)((T + 63) / 64), (unsigned)((E + 16 * NEB - 1) / (16 * NEB)), (unsigned)ns);
    router_gemm_kernel<NEB><<<grid, 256, 0, s>>>(T, d, E, router_kspan(d, ns), x, wrt, out);
}

hipError_t launch_router(int T, int d, int E, int K, int dtype, int flags, const void* x,
                         const void* w_router, const float* bias, float* logits, float* probs,
                         float* prob_sum, int32_t* ids, float* w, void* ws, hipStream_t s,
                         float* loss_part) {
    const RouterLayout L = router_layout(T, d, E, dtype);
    char* base = reinterpret_cast<char*>(ws);
    float* part = prob_sum ? reinterpret_cast<float*>(base + L.psum) : nullptr;
    hipError_t err;
    int nsplit = 1;
    const float* src = logits;
    float* logits_out = nullptr;
    if (x != nullptr && dtype == MOE_DTYPE_BF16) {
        bf16* wrt = reinterpret_cast<bf16*>(base + L.wrt);
        dim3 tg((unsigned)((d + 63) / 64), (unsigned)((E + 63) / 64));
        router_transpose_kernel<<<tg, 256, 0, s>>>(d, E, (const bf16*)w_router, wrt);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        nsplit = L.ns;
        float* gout = nsplit > 1 ? reinterpret_cast<float*>(base + L.part) : logits;
        switch (router_neb(E)) {
            case 1: launch_gemm_t<1>(T, d, E, nsplit, (const bf16*)x, wrt, gout, s); break;
            case 2: launch_gemm_t<2>(T, d, E, nsplit, (const bf16*)x, wrt, gout, s); break;
            case 4: launch_gemm_t<4>(T, d, E, nsplit, (const bf16*)x, wrt, gout, s); break;
            default: launch_gemm_t<8>(T, d, E, nsplit, (const bf16*)x, wrt, gout, s); break;
        }
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if (nsplit > 1) {
            src = gout;
            logits_out = logits;
        }
    } else if (x != nullptr) {  // fp32 scores
        const size_t n = (size_t)T * E;
        router_logits_f32_kernel<<<(unsigned)((n + 3) / 4), 256, 0, s>>>(
            T, d, E, (const float*)x, (const float*)w_router, logits);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    err = launch_route(T, E, K, flags, nsplit, src, logits_out, bias, probs, part, loss_part, ids, w, s);
    if (err != hipSuccess || !prob_sum) return err;
    psum_reduce_kernel<<<E, 256, 0, s>>>(router_num_blocks(T, E), E, part, prob_sum);
    return hipGetLastError();
}

}  // namespace moe
