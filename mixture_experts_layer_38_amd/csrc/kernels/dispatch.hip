// Dispatch: group the (token, slot) assignments per expert and gather the
// token rows into one contiguous block per expert.  MoE notes
// (www.cf-1.com/news/5905749) §2.1 (regroup tokens per expert with a sort and a
// cumulative sum) and §3.1 (a per-expert capacity truncates the overflow).
//
// Four kernels, none of which lets an atomic decide an order:
//   count   : each block histograms a contiguous chunk of the flat assignment
//             list t*K+k into LDS (integer adds commute, so the counts are exact);
//   scan    : one block turns the per-block counts into per-block bases (in
//             block order), totals, kept = min(count, C) and offsets = exscan(kept);
//   scatter : one wave per chunk walks it in rounds of 64 in flat order; lanes
//             that hold the same expert find each other with ballots over the
//             bits of the id (a wave multi-split), so each assignment's rank is
//             base + earlier lanes with that id; the last lane of the group
//             advances the per-expert base in LDS;
//   gather  : one wave per grouped row copies x[t] with 16-byte loads.
// Up to DS_SMALL_MAX assignments (decode-sized batches), count, scan and
// scatter run as one workgroup instead (same arithmetic, one launch).
#include "../device_common.h"
#include "../launch.h"
#include "dispatch_small.h"

namespace moe {

constexpr int DS_THREADS = 256;

// Chunk of the flat assignment list per count block / scatter wave: small
// enough that the scatter's serial rounds stay few, large enough that the scan
// over blocks stays short.
static int dispatch_chunk(int n) {
    int ch = 256;
    while ((n + ch - 1) / ch > 2048) ch *= 2;
    return ch;
}
static int dispatch_blocks(int n) {
    const int ch = dispatch_chunk(n);
    const int b = (n + ch - 1) / ch;
    return b > 0 ? b : 1;
}

size_t dispatch_ws_bytes(int T, int K, int E) {
    const int n = T * K;
    return align_up((size_t)dispatch_blocks(n) * E * sizeof(int32_t), 256);
}

__global__ __launch_bounds__(DS_THREADS) void dispatch_count_kernel(int n, int E, int ch,
                                                                   const int32_t* __restrict__ ids,
                                                                   int32_t* __restrict__ blk_counts) {
    extern __shared__ int hist[];
    for (int e = threadIdx.x; e < E; e += DS_THREADS) hist[e] = 0;
    __syncthreads();
    const int beg = blockIdx.x * ch;
    const int end = min(n, beg + ch);
    for (int i = beg + threadIdx.x; i < end; i += DS_THREADS) {
        const int e = ids[i];
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += DS_THREADS) blk_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// One block of 1024 threads; thread e owns expert e (E <= 1024).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(int nblk, int E, int capacity,
                                                            int32_t* __restrict__ blk,
                                                            int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ kept,
                                                            int32_t* __restrict__ offsets) {
    __shared__ int wave_tot[1024 / kWave];
    const int e = threadIdx.x;
    const int lane = e & (kWave - 1);
    const int wv = e / kWave;
    int run = 0;
    if (e < E) {
        // loads issued 16 at a time, then the running sum in block order
        for (int b0 = 0; b0 < nblk; b0 += 16) {
            int c[16];
#pragma unroll
            for (int q = 0; q < 16; ++q) c[q] = b0 + q < nblk ? blk[(size_t)(b0 + q) * E + e] : 0;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                if (b0 + q < nblk) blk[(size_t)(b0 + q) * E + e] = run;  // exclusive base of block b for expert e
                run += c[q];
            }
        }
        counts[e] = run;
    }
    const int kp = (e < E) ? (capacity < 0 ? run : min(run, capacity)) : 0;
    if (e < E) kept[e] = kp;
    int incl = kp;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) wave_tot[wv] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wv; ++w) before += wave_tot[w];
    const int excl = before + incl - kp;
    if (e < E) offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + kp;
}

__global__ __launch_bounds__(kWave) void dispatch_scatter_kernel(
    int n, int E, int nbits, int ch, int capacity, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ blk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ assign_row, int32_t* __restrict__ row_assign) {
    extern __shared__ int run[];  // running rank base per expert for this chunk
    const int lane = threadIdx.x;
    for (int e = lane; e < E; e += kWave) run[e] = blk_base[(size_t)blockIdx.x * E + e];
    __syncthreads();
    const int S = offsets[E];
    const int beg = blockIdx.x * ch;
    const int end = min(n, beg + ch);
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int base = beg; base < end; base += kWave) {
        const int i = base + lane;
        const bool in = i < end;
        const int e = in ? ids[i] : -1;
        const bool ok = in && (unsigned)e < (unsigned)E;
        unsigned long long peers = __ballot(ok);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = ok && ((e >> b) & 1);
            const unsigned long long bb = __ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        if (ok) {
            const int r0 = run[e];
            const int rank = r0 + __popcll(peers & below);
            const int last = 63 - __clzll(peers);
            if (capacity < 0 || rank < capacity) {
                const int row = offsets[e] + rank;
                assign_row[i] = row;
                if ((unsigned)row < (unsigned)n) row_assign[row] = i;
            } else {
                assign_row[i] = -1;
            }
            if (lane == last) run[e] = r0 + __popcll(peers);
        } else if (in) {
            assign_row[i] = -1;
        }
    }
    // Rows past the kept total S carry no assignment.
    for (int j = max(beg, S) + lane; j < end; j += kWave) row_assign[j] = -1;
}

// count + scan + scatter of at most DS_SMALL_MAX assignments in one block of
// 1024 threads.
__global__ __launch_bounds__(1024) void dispatch_small_kernel(
    int n, int E, int nbits, int capacity, const int32_t* __restrict__ ids,
    int32_t* __restrict__ counts, int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
    int32_t* __restrict__ assign_row, int32_t* __restrict__ row_assign) {
    __shared__ int hist[1024];
    __shared__ int offs[1024];
    __shared__ int wave_tot[1024 / kWave];
    dispatch_small_block(n, E, nbits, capacity, ids, counts, kept, offsets, assign_row, row_assign, hist,
                         offs, wave_tot);
}

__global__ __launch_bounds__(DS_THREADS) void dispatch_gather_kernel(
    int T, int K, int row_bytes, const int32_t* __restrict__ total,
    const int32_t* __restrict__ row_assign, const char* __restrict__ x, char* __restrict__ x_perm) {
    const int S = min(*total, T * K);
    const int row = blockIdx.x * (DS_THREADS / kWave) + (int)(threadIdx.x / kWave);
    if (row >= S) return;
    const int lane = lane_id();
    const int src = row_assign[row] / K;
    if ((unsigned)src >= (unsigned)T) return;
    const char* s = x + (size_t)src * row_bytes;
    char* dst = x_perm + (size_t)row * row_bytes;
    for (int off = lane * 16; off < row_bytes; off += kWave * 16) store16(dst + off, load16(s + off));
}

hipError_t launch_dispatch(int T, int K, int E, int d, int dtype, int capacity,
                           const int32_t* ids, const void* x, int32_t* counts, int32_t* kept,
                           int32_t* offsets, int32_t* assign_row, int32_t* row_assign,
                           void* x_perm, void* ws, hipStream_t s) {
    const int n = T * K;
    const int ch = dispatch_chunk(n);
    const int nblk = dispatch_blocks(n);
    int32_t* blk = reinterpret_cast<int32_t*>(ws);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    hipError_t err;
    if (n <= DS_SMALL_MAX) {
        MOE_TIMED_LAUNCH(MOE_KERNEL_DISPATCH_SCATTER, s,
                         dispatch_small_kernel<<<1, 1024, 0, s>>>(n, E, nbits, capacity, ids, counts,
                                                                  kept, offsets, assign_row, row_assign));
        if ((err = hipGetLastError()) != hipSuccess) return err;
    } else {
        MOE_TIMED_LAUNCH(MOE_KERNEL_DISPATCH_COUNT, s,
                         dispatch_count_kernel<<<nblk, DS_THREADS, (size_t)E * 4, s>>>(n, E, ch, ids, blk));
        if ((err = hipGetLastError()) != hipSuccess) return err;
        MOE_TIMED_LAUNCH(MOE_KERNEL_DISPATCH_SCAN, s,
                         dispatch_scan_kernel<<<1, 1024, 0, s>>>(nblk, E, capacity, blk, counts, kept, offsets));
        if ((err = hipGetLastError()) != hipSuccess) return err;
        MOE_TIMED_LAUNCH(MOE_KERNEL_DISPATCH_SCATTER, s,
                         dispatch_scatter_kernel<<<nblk, kWave, (size_t)E * 4, s>>>(
                             n, E, nbits, ch, capacity, ids, blk, offsets, assign_row, row_assign));
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if (x == nullptr) return hipSuccess;
    const int esz = dtype == MOE_DTYPE_F32 ? 4 : 2;
    const int rows_per_block = DS_THREADS / kWave;
    const unsigned grid = (unsigned)((n + rows_per_block - 1) / rows_per_block);
    MOE_TIMED_LAUNCH(MOE_KERNEL_DISPATCH_GATHER, s,
                     dispatch_gather_kernel<<<grid, DS_THREADS, 0, s>>>(
                         T, K, d * esz, offsets + E, row_assign, (const char*)x, (char*)x_perm));
    return hipGetLastError();
}

}  // namespace moe
