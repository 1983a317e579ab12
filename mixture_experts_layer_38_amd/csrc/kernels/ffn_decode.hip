// Grouped SwiGLU FFN for small expert groups (decode): MoE notes
// (www.cf-1.com/news/5905749) §2 step 3; the engineering page
// (ybb.press/quantum-computing/18594) §2.3 notes that decode is bound by
// loading expert weights, which is what this kernel is shaped for.
//
// Each workgroup owns a strip of 16 R weight rows of one expert (for gate/up
// the same rows of W1 and of W3) and its four waves split the reduction
// dimension.  A wave streams its rows in chunks of 128 * CPI k values.  In a
// chunk, load instruction s reads bytes [64 s, 64 s + 64) of the chunk of every
// row: the four lanes of a row read 64 contiguous bytes, and the 4 * CPI
// instructions cover the chunk.  The k positions fed to the 16x16x32 MFMAs
// follow the same permutation for the weight and for the token operand, so the
// contraction is unchanged.  Weights are read once with plain loads (on gfx950
// the non-temporal hint measured slower for this stream) and double-buffered
// in registers.  The expert's tokens (the second operand, 16 * NCB per pass;
// an expert with more rows takes several passes over its weights) are read
// from L2 just before their use.  Partial sums meet in LDS, where the
// fixed-order sum and the epilogue (SiLU(g1) * g3 for gate/up) run.  Experts
// with no rows are skipped without touching their weights.
#include <algorithm>

#include "../device_common.h"
#include "../launch.h"

namespace moe {

constexpr int DC_ROWS = 16;
constexpr int DC_WAVES = 4;
constexpr int DC_KCH = 128;

// 16 bytes at row[k .. k+8) when k < K, else zeros.  The load itself is
// unconditional (at a clamped, valid address) and the zeros come from a
// select, so the compiler emits no branch around it and can keep exact
// counts of the loads in flight.  K is a positive multiple of 8.
__device__ __forceinline__ u32x4 load16_masked(const bf16* row, int k, int K) {
    const u32x4 v = *(const u32x4*)(row + min(k, K - 8));
    const u32x4 z = {0u, 0u, 0u, 0u};
    return k < K ? v : z;
}

// The rows of expert e against this workgroup's strip of weight rows.
// K is the reduction length; lda and ldw are the row strides of A and of the
// weights (larger than K when the caller splits the reduction).  offsets may
// be NULL: then the group is rows [0, n_rows).  PART writes the fp32 sums to
// part [n_rows, N] instead of bf16 to out.  ZNEG reads row r of the group
// from A row rowmap[r * topk] as is, or as zeros when that entry is negative
// (the slots of a concatenation); otherwise row r is A row
// rowmap[r] / topk (rowmap NULL: row r).
template <bool GATED, int CPI, int NCB, bool ALIGNED, int R, bool PART = false, bool ZNEG = false>
__device__ __forceinline__ void ffn_decode_group(
    int e, int n_rows, int N, int K, const bf16* __restrict__ A, const int32_t* __restrict__ rowmap, int topk,
    const int32_t* __restrict__ offsets, const bf16* __restrict__ Wa, const bf16* __restrict__ Wb,
    bf16* __restrict__ out, int lda, int ldw, float* __restrict__ part = nullptr) {
    constexpr int NG = GATED ? 2 : 1;
    constexpr int NS = 4 * CPI;          // 32-wide slices per chunk
    constexpr int KCH = DC_KCH * CPI;  // k per chunk
    __shared__ float red[DC_WAVES - 1][R][NCB][NG][4][kWave];
    const int n0 = blockIdx.x * DC_ROWS * R;
    const int r0 = offsets ? offsets[e] : 0;
    const int m = (offsets ? min(offsets[e + 1], n_rows) : n_rows) - r0;
    if (r0 < 0 || m <= 0) return;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid & (kWave - 1);
    const int rl = lane & 15;
    const int g = lane >> 4;
    const int nch = (K + KCH - 1) / KCH;
    const int per = (nch + DC_WAVES - 1) / DC_WAVES;
    const int c_beg = min(nch, wave * per);
    const int c_end = min(nch, c_beg + per);
    const bf16* wa[R];
    const bf16* wb[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int wrow = min(n0 + DC_ROWS * r + rl, N - 1);
        wa[r] = Wa + ((size_t)e * N + wrow) * ldw;
        wb[r] = GATED ? Wb + ((size_t)e * N + wrow) * ldw : nullptr;
    }
    const int kl = g * 8;  // this lane's k offset inside each 32-wide slice

    for (int p0 = 0; p0 < m; p0 += 16 * NCB) {
        const int mp = min(m - p0, 16 * NCB);
        const int ncb = (mp + 15) / 16;
        f32x4 acc[R][NCB][NG];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) acc[r][cb][gi] = f32x4{0.f, 0.f, 0.f, 0.f};
        const bf16* arow[NCB];
        bool azero[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int r = r0 + p0 + min(cb * 16 + rl, mp - 1);
            if (ZNEG) {
                // a dropped slot never touches A: its (discarded) loads read
                // the first weight row of the strip, which spans the same k
                const int a = rowmap[(size_t)r * topk];
                azero[cb] = a < 0;
                arow[cb] = a < 0 ? wa[0] : A + (size_t)a * lda;
            } else {
                azero[cb] = false;
                arow[cb] = A + (size_t)src_row(rowmap, topk, r) * lda;
            }
        }

        // Double buffer in registers: the weight loads of chunk c + 1 are issued
        // after the token loads of chunk c, so waiting for the tokens of chunk c
        // (and the weights of chunk c, issued one step earlier) leaves chunk
        // c + 1 in flight while chunk c is multiplied.
        u32x4 wc[R][NG][NS], wn[R][NG][NS];
        auto load_w = [&](int c, u32x4 (&wd)[R][NG][NS]) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const int k = c * KCH + s * 32 + kl;
                    if (ALIGNED) {  // K is a multiple of the chunk: every load is in range
                        wd[r][0][s] = load16(wa[r] + k);
                        if (GATED) wd[r][NG - 1][s] = load16(wb[r] + k);
                    } else {
                        wd[r][0][s] = load16_masked(wa[r], k, K);
                        if (GATED) wd[r][NG - 1][s] = load16_masked(wb[r], k, K);
                    }
                }
        };
        if (c_beg < c_end) load_w(c_beg, wc);
        for (int c = c_beg; c < c_end; ++c) {
            u32x4 xv[NCB][NS];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (NCB == 1 || cb < ncb) {
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        const int k = c * KCH + s * 32 + kl;
                        xv[cb][s] = ALIGNED ? load16(arow[cb] + k) : load16_masked(arow[cb], k, K);
                        if (ZNEG) xv[cb][s] = azero[cb] ? u32x4{0u, 0u, 0u, 0u} : xv[cb][s];
                    }
                }
            }
            if (c + 1 < c_end) load_w(c + 1, wn);
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if (NCB == 1 || cb < ncb) {
#pragma unroll
                    for (int s = 0; s < NS; ++s) {
                        const bf16x8 xb = as_bf16x8(xv[cb][s]);
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            acc[r][cb][0] = mfma16(as_bf16x8(wc[r][0][s]), xb, acc[r][cb][0]);
                            if (GATED)
                                acc[r][cb][NG - 1] = mfma16(as_bf16x8(wc[r][NG - 1][s]), xb, acc[r][cb][NG - 1]);
                        }
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                    for (int s = 0; s < NS; ++s) wc[r][gi][s] = wn[r][gi][s];
        }
        if (wave > 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
                        for (int i = 0; i < 4; ++i) red[wave - 1][r][cb][gi][i][lane] = acc[r][cb][gi][i];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    if (cb >= ncb) break;
                    // lane holds output (weight row 4g + i of block r, token column rl)
                    const int tcol = cb * 16 + rl;
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float s0 = acc[r][cb][0][i];
                        float s1 = GATED ? acc[r][cb][NG - 1][i] : 0.0f;
#pragma unroll
                        for (int w = 0; w < DC_WAVES - 1; ++w) {
                            s0 += red[w][r][cb][0][i][lane];
                            if (GATED) s1 += red[w][r][cb][NG - 1][i][lane];
                        }
                        v[i] = GATED ? silu(s0) * s1 : s0;
                    }
                    if (PART && tcol < mp) {
                        // N is a multiple of 4 here (the caller checks), so
                        // the four values are one aligned 16-byte store
                        const int col = n0 + DC_ROWS * r + g * 4;
                        if (col < N)
                            *reinterpret_cast<f32x4*>(part + (size_t)(r0 + p0 + tcol) * N + col) =
                                f32x4{v[0], v[1], v[2], v[3]};
                    } else if (tcol < mp) {
                        const int col = n0 + DC_ROWS * r + g * 4;
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
        }
        __syncthreads();
    }
}

template <bool GATED, int CPI, int NCB, bool ALIGNED, int R>
__global__ __launch_bounds__(DC_WAVES * kWave) void ffn_decode_kernel(
    int n_rows, int N, int K, const bf16* __restrict__ A, const int32_t* __restrict__ rowmap, int topk,
    const int32_t* __restrict__ offsets, const bf16* __restrict__ Wa, const bf16* __restrict__ Wb,
    bf16* __restrict__ out) {
    ffn_decode_group<GATED, CPI, NCB, ALIGNED, R>(blockIdx.y, n_rows, N, K, A, rowmap, topk, offsets, Wa, Wb, out,
                                                  K, K);
}

// Expert blockIdx.y of a decode-sized batch: its rows in passes of 16 token
// rows (one token block, CPI1 chunks per iteration) when it holds at most 16,
// else in passes of 32 (two token blocks, CPI2 chunks), so that an expert
// with 17-32 rows streams its weights once and one with 33-64 rows twice
// instead of four times.  The two paths are chosen per workgroup; a kernel
// holding both takes the registers of the larger, so CPI2 is picked to keep
// that within the single path's occupancy.
template <bool GATED, int CPI1, int CPI2, bool ALIGNED, int R, bool FOUR = false>
__global__ __launch_bounds__(DC_WAVES * kWave) void ffn_decode_expert_kernel(
    int n_rows, int N, int K, const bf16* __restrict__ A, const int32_t* __restrict__ rowmap, int topk,
    const int32_t* __restrict__ offsets, const bf16* __restrict__ Wa, const bf16* __restrict__ Wb,
    bf16* __restrict__ out) {
    const int e = blockIdx.y;
    const int m = min(offsets[e + 1], n_rows) - offsets[e];
    if (m <= DC_ROWS)
        ffn_decode_group<GATED, CPI1, 1, ALIGNED, R>(e, n_rows, N, K, A, rowmap, topk, offsets, Wa, Wb, out, K, K);
    else if (!FOUR || m <= 2 * DC_ROWS)
        ffn_decode_group<GATED, CPI2, 2, ALIGNED, R>(e, n_rows, N, K, A, rowmap, topk, offsets, Wa, Wb, out, K, K);
    else
        ffn_decode_group<GATED, 1, 4, ALIGNED, R>(e, n_rows, N, K, A, rowmap, topk, offsets, Wa, Wb, out, K, K);
}

// The experts listed in elist[0 .. *ecount) (small groups of a large batch),
// taken in turn by the gridDim.y workgroups of each strip; like the decode
// kernel, an expert of at most 16 rows runs in passes of one token block
// (CPI1 chunks per iteration), a larger one in passes of two (CPI2).
template <bool GATED, int CPI1, int CPI2, bool ALIGNED, int R>
__global__ __launch_bounds__(DC_WAVES * kWave) void ffn_small_experts_kernel(
    int n_rows, int N, int K, const bf16* __restrict__ A, const int32_t* __restrict__ rowmap, int topk,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ elist, const int32_t* __restrict__ ecount,
    const bf16* __restrict__ Wa, const bf16* __restrict__ Wb, bf16* __restrict__ out) {
    const int cnt = *ecount;
    for (int i = blockIdx.y; i < cnt; i += gridDim.y) {
        const int e = elist[i];
        const int m = min(offsets[e + 1], n_rows) - offsets[e];
        if (m <= DC_ROWS)
            ffn_decode_group<GATED, CPI1, 1, ALIGNED, R>(e, n_rows, N, K, A, rowmap, topk, offsets, Wa, Wb, out, K,
                                                         K);
        else
            ffn_decode_group<GATED, CPI2, 2, ALIGNED, R>(e, n_rows, N, K, A, rowmap, topk, offsets, Wa, Wb, out, K,
                                                         K);
    }
}

template <bool ALIGNED>
static hipError_t launch_decode_t(int n_rows, int E, int d, int F, const void* A,
                                  const int32_t* rowmap, int topk, const int32_t* offsets,
                                  const void* w1, const void* w3, const void* w2, void* act,
                                  void* h, hipStream_t s) {
    dim3 g1((F + DC_ROWS - 1) / DC_ROWS, E);
    // Two 128-wide chunks per iteration when they tile d exactly (more weight
    // bytes in flight per wave: 0.35% faster on the Mixtral-shaped decode
    // batch); the two-block path of experts with more than 16 rows takes one
    // (with two, the kernel's 270 registers would halve its occupancy).
    // (two is set only on the aligned path, which the launch below assumes)
    bool two = false;
    if constexpr (ALIGNED) two = d % (2 * DC_KCH) == 0;
    if (two)
        MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_GATE_UP, s,
                         ffn_decode_expert_kernel<true, 2, 1, true, 1, true><<<g1, DC_WAVES * kWave, 0, s>>>(
                             n_rows, F, d, (const bf16*)A, rowmap, topk, offsets, (const bf16*)w1,
                             (const bf16*)w3, (bf16*)act));
    else
        MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_GATE_UP, s,
                         ffn_decode_expert_kernel<true, 1, 1, ALIGNED, 1, true><<<g1, DC_WAVES * kWave, 0, s>>>(
                             n_rows, F, d, (const bf16*)A, rowmap, topk, offsets, (const bf16*)w1,
                             (const bf16*)w3, (bf16*)act));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // Four 16-row blocks per workgroup for the down projection: each token
    // fragment (an L2 read of the long activation rows) feeds four MFMAs; two
    // 128-wide chunks per iteration when they tile F exactly.  Measured on the
    // Mixtral-shaped decode batch (per layer, each against two blocks with two
    // chunks on the same box): four blocks with one chunk 2.75 us slower, four
    // blocks with two chunks 0.6 us faster, two blocks with four chunks
    // 2.75 us slower; with one chunk, one block was 26 us slower than two and
    // four 1.7 us faster.
    dim3 g2((d + 4 * DC_ROWS - 1) / (4 * DC_ROWS), E);
    bool two_f = false;
    if constexpr (ALIGNED) two_f = F % (2 * DC_KCH) == 0;
    if (two_f)
        MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_DOWN, s,
                         ffn_decode_expert_kernel<false, 2, 2, true, 4><<<g2, DC_WAVES * kWave, 0, s>>>(
                             n_rows, d, F, (const bf16*)act, nullptr, 1, offsets, (const bf16*)w2, nullptr,
                             (bf16*)h));
    else
        MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_DOWN, s,
                         ffn_decode_expert_kernel<false, 1, 1, ALIGNED, 4><<<g2, DC_WAVES * kWave, 0, s>>>(
                             n_rows, d, F, (const bf16*)act, nullptr, 1, offsets, (const bf16*)w2, nullptr,
                             (bf16*)h));
    return hipGetLastError();
}

// Experts with at most DC_SMALL_ROWS rows inside a larger batch (listed by the
// tile plan): one pass of 16 or 32 token rows over each weight row, so every
// weight byte is read once; gy = min(E, 64) workgroups per strip take the
// experts in turn.
template <bool ALIGNED>
static hipError_t launch_small_experts_t(bool gated, int gy, int n_rows, int N, int K, const void* A,
                                         const int32_t* rowmap, int topk, const int32_t* offsets,
                                         const int32_t* elist, const int32_t* ecount, const void* wa,
                                         const void* wb, void* out, hipStream_t s) {
    // two 128-wide chunks per iteration on the one-block path when they tile K
    bool two = false;
    if constexpr (ALIGNED) two = K % (2 * DC_KCH) == 0;
    if (gated) {
        dim3 g((N + DC_ROWS - 1) / DC_ROWS, gy);
        if (two)
            ffn_small_experts_kernel<true, 2, 1, true, 1><<<g, DC_WAVES * kWave, 0, s>>>(
                n_rows, N, K, (const bf16*)A, rowmap, topk, offsets, elist, ecount, (const bf16*)wa,
                (const bf16*)wb, (bf16*)out);
        else
            ffn_small_experts_kernel<true, 1, 1, ALIGNED, 1><<<g, DC_WAVES * kWave, 0, s>>>(
                n_rows, N, K, (const bf16*)A, rowmap, topk, offsets, elist, ecount, (const bf16*)wa,
                (const bf16*)wb, (bf16*)out);
    } else {
        dim3 g((N + 2 * DC_ROWS - 1) / (2 * DC_ROWS), gy);
        if (two)
            ffn_small_experts_kernel<false, 2, 1, true, 2><<<g, DC_WAVES * kWave, 0, s>>>(
                n_rows, N, K, (const bf16*)A, nullptr, 1, offsets, elist, ecount, (const bf16*)wa, nullptr,
                (bf16*)out);
        else
            ffn_small_experts_kernel<false, 1, 1, ALIGNED, 2><<<g, DC_WAVES * kWave, 0, s>>>(
                n_rows, N, K, (const bf16*)A, nullptr, 1, offsets, elist, ecount, (const bf16*)wa, nullptr,
                (bf16*)out);
    }
    return hipGetLastError();
}

hipError_t launch_small_experts(bool gated, int E, int n_rows, int N, int K, const void* A,
                                const int32_t* rowmap, int topk, const int32_t* offsets, const int32_t* elist,
                                const int32_t* ecount, const void* wa, const void* wb, void* out, hipStream_t s) {
    const int gy = E < 64 ? E : 64;
    if (K % DC_KCH == 0)
        return launch_small_experts_t<true>(gated, gy, n_rows, N, K, A, rowmap, topk, offsets, elist, ecount, wa,
                                            wb, out, s);
    return launch_small_experts_t<false>(gated, gy, n_rows, N, K, A, rowmap, topk, offsets, elist, ecount, wa,
                                         wb, out, s);
}

// One group of at most 64 rows against W [N, K]: one pass of 64 token rows
// over each strip of 32 weight rows.  With few strips the reduction is split
// into gridDim.y parts of kp values (a multiple of the 128-value chunk), each
// writing fp32 sums to its own slice of part; linear_part_reduce_kernel then
// adds the parts in index order, so the result does not depend on timing.
// NCB 16-row token blocks per pass: 2 for up to 32 rows (fewer registers,
// three workgroups per CU), 4 for up to 64.
template <bool ALIGNED, int NCB>
__global__ __launch_bounds__(DC_WAVES * kWave) void linear_part_kernel(
    int n_rows, int N, int K, int kp, const bf16* __restrict__ A, const int32_t* __restrict__ offs,
    const bf16* __restrict__ W, float* __restrict__ part) {
    const int kb = blockIdx.y * kp;
    ffn_decode_group<false, 1, NCB, ALIGNED, 2, true>(0, n_rows, N, min(kp, K - kb), A + kb, nullptr, 1, offs,
                                                      W + kb, nullptr, nullptr, K, K,
                                                      part + (size_t)blockIdx.y * n_rows * N);
}

// Concatenation combine for at most 64 tokens (MoE notes §2.3): part p of
// the reduction over W_cat [d, Ks d] covers columns [c0, c0 + kp) of slot
// j = p / qs (c0 = (p % qs) kp), so its token rows are the grouped expert
// rows h[assign_row[t Ks + j]] read in place (a dropped slot reads as zeros)
// and no concatenated copy is built.
template <bool ALIGNED, int NCB>
__global__ __launch_bounds__(DC_WAVES * kWave) void concat_part_kernel(
    int T, int d, int Ks, int kp, int qs, const bf16* __restrict__ h, const int32_t* __restrict__ assign_row,
    const bf16* __restrict__ W, float* __restrict__ part) {
    const int j = blockIdx.y / qs;
    const int c0 = (blockIdx.y - j * qs) * kp;
    ffn_decode_group<false, 1, NCB, ALIGNED, 2, true, true>(0, T, d, min(kp, d - c0), h + c0, assign_row + j, Ks,
                                                            nullptr, W + (size_t)j * d + c0, nullptr, nullptr, d,
                                                            Ks * d, part + (size_t)blockIdx.y * T * d);
}

__global__ __launch_bounds__(256) void linear_part_reduce_kernel(int n, int parts, const float* __restrict__ part,
                                                                 bf16* __restrict__ y) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) {
        float v = part[i];
        for (int j = 1; j < parts; ++j) v += part[(size_t)j * n + i];
        y[i] = (bf16)v;
    }
}

// Parts of the reduction for a decode-sized linear layer: enough workgroups
// to keep every CU streaming weights (about 1024), each wave keeping at least
// eight chunks (shorter streams measured slower: a 64 MB weight took 20 us in
// two parts of eight chunks per wave and 22 us in eight parts of two).
// Returns the part length in *kp.
static int linear_parts(int N, int K, int* kp) {
    *kp = K;
    if (N % 4 != 0) return 1;
    const int gx = (N + 2 * DC_ROWS - 1) / (2 * DC_ROWS);
    const int nch = (K + DC_KCH - 1) / DC_KCH;
    int parts = std::min(std::min((1024 + gx - 1) / gx, nch / (8 * DC_WAVES)), LIN_MAX_PARTS);
    if (parts < 1) parts = 1;
    *kp = ((nch + parts - 1) / parts) * DC_KCH;
    return (K + *kp - 1) / *kp;
}

size_t linear_small_ws_bytes(int n_rows, int N, int K) {
    int kp;
    const int parts = linear_parts(N, K, &kp);
    return parts > 1 ? (size_t)parts * n_rows * N * sizeof(float) : 0;
}

hipError_t launch_linear_small(int n_rows, int N, int K, const void* A, const int32_t* offs, const void* w,
                               void* out, void* ws, hipStream_t s) {
    int kp;
    const int parts = linear_parts(N, K, &kp);
    if (parts > 1) {
        dim3 g((N + 2 * DC_ROWS - 1) / (2 * DC_ROWS), parts);
        float* part = reinterpret_cast<float*>(ws);
        const bf16* a = (const bf16*)A;
        const bf16* wt = (const bf16*)w;
        const bool al = K % DC_KCH == 0;
        if (n_rows <= 32) {
            if (al) linear_part_kernel<true, 2><<<g, DC_WAVES * kWave, 0, s>>>(n_rows, N, K, kp, a, offs, wt, part);
            else linear_part_kernel<false, 2><<<g, DC_WAVES * kWave, 0, s>>>(n_rows, N, K, kp, a, offs, wt, part);
        } else {
            if (al) linear_part_kernel<true, 4><<<g, DC_WAVES * kWave, 0, s>>>(n_rows, N, K, kp, a, offs, wt, part);
            else linear_part_kernel<false, 4><<<g, DC_WAVES * kWave, 0, s>>>(n_rows, N, K, kp, a, offs, wt, part);
        }
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        const int n = n_rows * N;
        linear_part_reduce_kernel<<<std::max(1, std::min((n + 255) / 256, 1024)), 256, 0, s>>>(n, parts, part,
                                                                                              (bf16*)out);
        return hipGetLastError();
    }
    dim3 g((N + 2 * DC_ROWS - 1) / (2 * DC_ROWS), 1);
    if (K % DC_KCH == 0)
        ffn_decode_kernel<false, 1, 4, true, 2><<<g, DC_WAVES * kWave, 0, s>>>(
            n_rows, N, K, (const bf16*)A, nullptr, 1, offs, (const bf16*)w, nullptr, (bf16*)out);
    else
        ffn_decode_kernel<false, 1, 4, false, 2><<<g, DC_WAVES * kWave, 0, s>>>(
            n_rows, N, K, (const bf16*)A, nullptr, 1, offs, (const bf16*)w, nullptr, (bf16*)out);
    return hipGetLastError();
}

// Parts per slot for the concatenation combine: the count the plain linear
// layer would use, spread over the Ks slots (at least one per slot); 0 when
// the concatenation is not decode-sized or would need more than
// LIN_MAX_PARTS parts (the caller then gathers the rows and uses
// launch_linear).
static int concat_parts_per_slot(int T, int Ks, int d, int* kp) {
    if (T > LIN_SMALL_ROWS || d % 4 != 0) return 0;
    int kpl;
    const int parts = linear_parts(d, Ks * d, &kpl);
    const int q = std::max(1, parts / Ks);
    if (Ks * q > LIN_MAX_PARTS) return 0;
    *kp = ((d + q - 1) / q + DC_KCH - 1) / DC_KCH * DC_KCH;
    return (d + *kp - 1) / *kp;
}

size_t concat_small_ws_bytes(int T, int Ks, int d) {
    int kp;
    const int qs = concat_parts_per_slot(T, Ks, d, &kp);
    return qs ? (size_t)Ks * qs * T * d * sizeof(float) : 0;
}

bool concat_small_ok(int T, int Ks, int d) {
    int kp;
    return concat_parts_per_slot(T, Ks, d, &kp) > 0;
}

hipError_t launch_concat_small(int T, int Ks, int d, const void* h, const int32_t* assign_row, const void* w_cat,
                               void* y, void* ws, hipStream_t s) {
    int kp;
    const int qs = concat_parts_per_slot(T, Ks, d, &kp);
    if (qs == 0) return hipErrorInvalidValue;
    const int parts = Ks * qs;
    dim3 g((d + 2 * DC_ROWS - 1) / (2 * DC_ROWS), parts);
    float* part = reinterpret_cast<float*>(ws);
    const bf16* hb = (const bf16*)h;
    const bf16* wt = (const bf16*)w_cat;
    const bool al = d % kp == 0 && kp % DC_KCH == 0;
    if (T <= 32) {
        if (al) concat_part_kernel<true, 2><<<g, DC_WAVES * kWave, 0, s>>>(T, d, Ks, kp, qs, hb, assign_row, wt, part);
        else concat_part_kernel<false, 2><<<g, DC_WAVES * kWave, 0, s>>>(T, d, Ks, kp, qs, hb, assign_row, wt, part);
    } else {
        if (al) concat_part_kernel<true, 4><<<g, DC_WAVES * kWave, 0, s>>>(T, d, Ks, kp, qs, hb, assign_row, wt, part);
        else concat_part_kernel<false, 4><<<g, DC_WAVES * kWave, 0, s>>>(T, d, Ks, kp, qs, hb, assign_row, wt, part);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int n = T * d;
    linear_part_reduce_kernel<<<std::max(1, std::min((n + 255) / 256, 1024)), 256, 0, s>>>(n, parts, part,
                                                                                          (bf16*)y);
    return hipGetLastError();
}

hipError_t launch_ffn_decode(int n_rows, int E, int d, int F, const void* A, const int32_t* rowmap,
                             int topk, const int32_t* offsets, const void* w1, const void* w3,
                             const void* w2, void* act, void* h, hipStream_t s) {
    if (d % DC_KCH == 0 && F % DC_KCH == 0)
        return launch_decode_t<true>(n_rows, E, d, F, A, rowmap, topk, offsets, w1, w3, w2, act, h, s);
    return launch_decode_t<false>(n_rows, E, d, F, A, rowmap, topk, offsets, w1, w3, w2, act, h, s);
}

}  // namespace moe
