// Grouped SwiGLU FFN for small expert groups (decode): MoE notes
// (www.cf-1.com/news/5905749) §2 step 3; the engineering page
// (ybb.press/quantum-computing/18594) §2.3 notes that decode is bound by
// loading expert weights, which is what this kernel is shaped for.
//
// Each workgroup owns a strip of 16 weight rows of one expert (for gate/up the
// same 16 rows of W1 and of W3) and its four waves split the reduction
// dimension.  A wave streams its rows in 128-wide k chunks: lane (r, g) loads 64
// contiguous bytes of row r (so the four lanes of a row read 256 contiguous
// bytes), and feeds them to four 16x16x32 MFMAs whose k positions are permuted
// identically for the weight and the token operand.  The expert's tokens (at
// most 32 per pass, two 16-column MFMA blocks) are the second operand, read
// from L2.  Partial sums meet in LDS, where the fixed-order sum and the epilogue
// (SiLU(g1) * g3 for gate/up) run.  Experts with no rows are skipped without
// touching their weights.
#include "../device_common.h"
#include "../launch.h"

namespace moe {

constexpr int DC_ROWS = 16;
constexpr int DC_WAVES = 4;
constexpr int DC_KCH = 128;
constexpr int DC_MAXCB = 2;

template <bool GATED>
__global__ __launch_bounds__(DC_WAVES * kWave) void ffn_decode_kernel(
    int n_rows, int N, int K, const bf16* __restrict__ A, const int32_t* __restrict__ offsets,
    const bf16* __restrict__ Wa, const bf16* __restrict__ Wb, bf16* __restrict__ out) {
    constexpr int NG = GATED ? 2 : 1;
    __shared__ float red[DC_WAVES][DC_MAXCB][NG][4][kWave];
    const int e = blockIdx.y;
    const int n0 = blockIdx.x * DC_ROWS;
    const int r0 = offsets[e];
    const int m = min(offsets[e + 1], n_rows) - r0;
    if (r0 < 0 || m <= 0) return;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const int rl = lane & 15;
    const int g = lane >> 4;
    const int nch = (K + DC_KCH - 1) / DC_KCH;
    const int per = (nch + DC_WAVES - 1) / DC_WAVES;
    const int c_beg = wave * per;
    const int c_end = min(nch, c_beg + per);
    const int wrow = min(n0 + rl, N - 1);
    const bf16* wa = Wa + ((size_t)e * N + wrow) * K;
    const bf16* wb = GATED ? Wb + ((size_t)e * N + wrow) * K : nullptr;

    for (int p0 = 0; p0 < m; p0 += 16 * DC_MAXCB) {
        const int mp = min(m - p0, 16 * DC_MAXCB);
        const int ncb = (mp + 15) / 16;
        f32x4 acc[DC_MAXCB][NG];
#pragma unroll
        for (int cb = 0; cb < DC_MAXCB; ++cb)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) acc[cb][gi] = f32x4{0.f, 0.f, 0.f, 0.f};
        const bf16* arow[DC_MAXCB];
#pragma unroll
        for (int cb = 0; cb < DC_MAXCB; ++cb)
            arow[cb] = A + (size_t)(r0 + p0 + min(cb * 16 + rl, mp - 1)) * K;

        for (int c = c_beg; c < c_end; ++c) {
            const int kb = c * DC_KCH + g * 32;
            u32x4 wv[4];
            u32x4 wv3[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k = kb + s * 8;
                wv[s] = load16_or_zero(wa + k, k < K);
                if (GATED) wv3[s] = load16_or_zero(wb + k, k < K);
            }
#pragma unroll
            for (int cb = 0; cb < DC_MAXCB; ++cb) {
                if (cb < ncb) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int k = kb + s * 8;
                        const bf16x8 xv = as_bf16x8(load16_or_zero(arow[cb] + k, k < K));
                        acc[cb][0] = mfma16(as_bf16x8(wv[s]), xv, acc[cb][0]);
                        if (GATED) acc[cb][NG - 1] = mfma16(as_bf16x8(wv3[s]), xv, acc[cb][NG - 1]);
                    }
                }
            }
        }
#pragma unroll
        for (int cb = 0; cb < DC_MAXCB; ++cb)
#pragma unroll
            for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[wave][cb][gi][i][lane] = acc[cb][gi][i];
        __syncthreads();
        if (wave == 0) {
            for (int cb = 0; cb < ncb; ++cb) {
                // lane holds output (weight row 4g + i, token column rl) of this block
                const int tcol = cb * 16 + rl;
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float s0 = red[0][cb][0][i][lane];
                    float s1 = GATED ? red[0][cb][NG - 1][i][lane] : 0.0f;
#pragma unroll
                    for (int w = 1; w < DC_WAVES; ++w) {
                        s0 += red[w][cb][0][i][lane];
                        if (GATED) s1 += red[w][cb][NG - 1][i][lane];
                    }
                    v[i] = GATED ? silu(s0) * s1 : s0;
                }
                if (tcol < mp) {
                    const int col = n0 + g * 4;
                    bf16* o = out + (size_t)(r0 + p0 + tcol) * N + col;
                    if (col + 3 < N) {
                        bf16x4 pk = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
                        *reinterpret_cast<bf16x4*>(o) = pk;
                    } else {
                        for (int i = 0; i < 4; ++i)
                            if (col + i < N) o[i] = (bf16)v[i];
                    }
                }
            }
        }
        __syncthreads();
    }
}

hipError_t launch_ffn_decode(int n_rows, int E, int d, int F, const void* x_perm, const int32_t* offsets,
                             const void* w1, const void* w3, const void* w2, void* act, void* h,
                             hipStream_t s) {
    dim3 g1((F + DC_ROWS - 1) / DC_ROWS, E);
    MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_GATE_UP, s,
                     ffn_decode_kernel<true><<<g1, DC_WAVES * kWave, 0, s>>>(
                         n_rows, F, d, (const bf16*)x_perm, offsets, (const bf16*)w1, (const bf16*)w3,
                         (bf16*)act));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    dim3 g2((d + DC_ROWS - 1) / DC_ROWS, E);
    MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_DOWN, s,
                     ffn_decode_kernel<false><<<g2, DC_WAVES * kWave, 0, s>>>(
                         n_rows, d, F, (const bf16*)act, offsets, (const bf16*)w2, nullptr, (bf16*)h));
    return hipGetLastError();
}

}  // namespace moe
