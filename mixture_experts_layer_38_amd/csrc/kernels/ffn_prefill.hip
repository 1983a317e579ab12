// Grouped SwiGLU FFN for large expert groups (prefill): MoE notes
// (www.cf-1.com/news/5905749) §2 step 3 and §2.3 (batched permute, then one
// batched GEMM per expert group); the engineering page
// (ybb.press/quantum-computing/18594) §2.3: prefill is compute-bound, so the
// GEMM throughput is what matters.
//
// Both GEMMs are "rows x weights^T" with both operands contiguous along the
// reduction dimension: act = SiLU(X W1^T) * (X W3^T) and h = act W2^T.
// A device-side plan (one tiny kernel) cuts every expert's rows into 128-row
// tiles; the GEMM grid is (weight tiles) x (an upper bound on row tiles), and
// workgroups past the real tile count exit at once.  A workgroup computes a
// 128 x 128 output tile with four waves in a 2 x 2 grid, each wave 64 x 64 with
// 32x32x16 bf16 MFMAs (weights as the first operand so each lane ends up with
// four consecutive output columns of one token).  Operand tiles move HBM ->
// registers -> LDS (padded rows, double buffered, one barrier per 64-wide k
// step).  For gate/up the weight tile interleaves 32-row blocks of W1 and W3 of
// the same output columns, so the SiLU-gate epilogue is local to each wave.
#include "../device_common.h"
#include "../launch.h"

namespace moe {

constexpr int PF_BM = 128;
constexpr int PF_BN = 128;
constexpr int PF_BK = 64;
constexpr int PF_LDS = PF_BK + 8;  // padded LDS row length (bf16)
constexpr int PF_THREADS = 256;

int prefill_max_mtiles(int n_rows, int E) { return n_rows / PF_BM + E + 1; }

// One block; thread e cuts expert e's rows into PF_BM-row tiles.
__global__ __launch_bounds__(1024) void ffn_plan_kernel(int E, int max_mt,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ mt_count,
                                                       int32_t* __restrict__ mt_expert,
                                                       int32_t* __restrict__ mt_row0) {
    __shared__ int wave_tot[1024 / kWave];
    const int e = threadIdx.x;
    const int lane = e & (kWave - 1);
    const int wv = e / kWave;
    const int rows = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (rows + PF_BM - 1) / PF_BM;
    int incl = nt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) wave_tot[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wv; ++w) before += wave_tot[w];
    const int start = before + incl - nt;
    if (e < E) {
        for (int j = 0; j < nt && start + j < max_mt; ++j) {
            mt_expert[start + j] = e;
            mt_row0[start + j] = offsets[e] + j * PF_BM;
        }
    }
    if (e == E - 1) *mt_count = min(start + nt, max_mt);
}

template <bool GATED>
__global__ __launch_bounds__(PF_THREADS) void ffn_prefill_kernel(
    int n_rows, int N, int K, const bf16* __restrict__ A, const int32_t* __restrict__ mt_count,
    const int32_t* __restrict__ mt_expert, const int32_t* __restrict__ mt_row0,
    const int32_t* __restrict__ offsets, const bf16* __restrict__ Wa, const bf16* __restrict__ Wb,
    bf16* __restrict__ out) {
    const int mt = blockIdx.y;
    if (mt >= *mt_count) return;
    const int e = mt_expert[mt];
    const int row0 = mt_row0[mt];
    const int row_end = min(offsets[e + 1], n_rows);
    const int nt = blockIdx.x;

    __shared__ __align__(16) bf16 sA[2][PF_BM * PF_LDS];
    __shared__ __align__(16) bf16 sB[2][PF_BN * PF_LDS];

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int lr = tid >> 3;        // 0..31: row within a 32-row slab
    const int lc = (tid & 7) * 8;   // 16-byte chunk within the 64-wide k step

    const bf16* a_src[4];
    const bf16* b_src[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = min(row0 + lr + 32 * j, n_rows - 1);
        a_src[j] = A + (size_t)r * K + lc;
        const int br = lr + 32 * j;
        if (GATED) {
            const int blk = br >> 5;
            const int f = min(nt * 64 + (blk >> 1) * 32 + (br & 31), N - 1);
            const bf16* W = (blk & 1) ? Wb : Wa;
            b_src[j] = W + ((size_t)e * N + f) * K + lc;
        } else {
            const int nr = min(nt * PF_BN + br, N - 1);
            b_src[j] = Wa + ((size_t)e * N + nr) * K + lc;
        }
    }

    const int nk = (K + PF_BK - 1) / PF_BK;
    u32x4 ra[4], rb[4];
    auto gload = [&](int kt) {
        const bool ok = kt * PF_BK + lc < K;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ra[j] = load16_or_zero(a_src[j] + (size_t)kt * PF_BK, ok);
            rb[j] = load16_or_zero(b_src[j] + (size_t)kt * PF_BK, ok);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            store16(&sA[buf][(lr + 32 * j) * PF_LDS + lc], ra[j]);
            store16(&sB[buf][(lr + 32 * j) * PF_LDS + lc], rb[j]);
        }
    };

    const int wm = wave & 1;   // token half of the tile
    const int wn = wave >> 1;  // weight half of the tile
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < PF_BK; ks += 16) {
            const int koff = ks + (lane >> 5) * 8;
            bf16x8 fw[2], ft[2];
#pragma unroll
            for (int wb = 0; wb < 2; ++wb)
                fw[wb] = *reinterpret_cast<const bf16x8*>(
                    &sB[cur][(wn * 64 + wb * 32 + (lane & 31)) * PF_LDS + koff]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
                ft[tb] = *reinterpret_cast<const bf16x8*>(
                    &sA[cur][(wm * 64 + tb * 32 + (lane & 31)) * PF_LDS + koff]);
#pragma unroll
            for (int wb = 0; wb < 2; ++wb)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) acc[wb][tb] = mfma32(fw[wb], ft[tb], acc[wb][tb]);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // acc[wb][tb][i]: weight row 8*(i/4) + 4*(lane/32) + i%4 of block wb,
    // token (lane % 32) of block tb.
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int grow = row0 + wm * 64 + tb * 32 + (lane & 31);
        if (grow >= row_end) continue;
        bf16* orow = out + (size_t)grow * N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int wr = 8 * q + 4 * (lane >> 5);
            if (GATED) {
                const int f = nt * 64 + wn * 32 + wr;
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = silu(acc[0][tb][4 * q + r]) * acc[1][tb][4 * q + r];
                if (f + 3 < N) {
                    bf16x4 pk = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
                    *reinterpret_cast<bf16x4*>(orow + f) = pk;
                } else {
                    for (int r = 0; r < 4; ++r)
                        if (f + r < N) orow[f + r] = (bf16)v[r];
                }
            } else {
#pragma unroll
                for (int wb = 0; wb < 2; ++wb) {
                    const int c = nt * PF_BN + wn * 64 + wb * 32 + wr;
                    const f32x16& a = acc[wb][tb];
                    if (c + 3 < N) {
                        bf16x4 pk = {(bf16)a[4 * q], (bf16)a[4 * q + 1], (bf16)a[4 * q + 2],
                                     (bf16)a[4 * q + 3]};
                        *reinterpret_cast<bf16x4*>(orow + c) = pk;
                    } else {
                        for (int r = 0; r < 4; ++r)
                            if (c + r < N) orow[c + r] = (bf16)a[4 * q + r];
                    }
                }
            }
        }
    }
}

size_t prefill_ws_bytes(int n_rows, int E) {
    return align_up((size_t)(1 + 2 * prefill_max_mtiles(n_rows, E)) * sizeof(int32_t), 256);
}

hipError_t launch_ffn_prefill(int n_rows, int E, int d, int F, const void* x_perm,
                              const int32_t* offsets, const void* w1, const void* w3,
                              const void* w2, void* act, void* h, void* ws, hipStream_t s) {
    const int max_mt = prefill_max_mtiles(n_rows, E);
    int32_t* mt_count = reinterpret_cast<int32_t*>(ws);
    int32_t* mt_expert = mt_count + 1;
    int32_t* mt_row0 = mt_expert + max_mt;
    MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_PLAN, s,
                     ffn_plan_kernel<<<1, 1024, 0, s>>>(E, max_mt, offsets, mt_count, mt_expert, mt_row0));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    dim3 g1((F + 63) / 64, max_mt);
    MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_GATE_UP, s,
                     ffn_prefill_kernel<true><<<g1, PF_THREADS, 0, s>>>(
                         n_rows, F, d, (const bf16*)x_perm, mt_count, mt_expert, mt_row0, offsets,
                         (const bf16*)w1, (const bf16*)w3, (bf16*)act));
    if ((err = hipGetLastError()) != hipSuccess) return err;
    dim3 g2((d + PF_BN - 1) / PF_BN, max_mt);
    MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_DOWN, s,
                     ffn_prefill_kernel<false><<<g2, PF_THREADS, 0, s>>>(
                         n_rows, d, F, (const bf16*)act, mt_count, mt_expert, mt_row0, offsets,
                         (const bf16*)w2, nullptr, (bf16*)h));
    return hipGetLastError();
}

}  // namespace moe
