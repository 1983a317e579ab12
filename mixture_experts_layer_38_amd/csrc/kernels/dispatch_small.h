// Single-workgroup dispatch of a small assignment list (decode-sized
// batches): histogram, capacity cut, exclusive scan and the stable scatter of
// the dispatch kernels, run by one block of 1024 threads.  Shared by the
// dispatch kernels and the fused small-batch router.
#pragma once

#include "../device_common.h"

namespace moe {

// The single workgroup walks the list in rounds of 64 with one wave (about half
// a microsecond per round); above this size the three-kernel dispatch is
// faster (measured at 4096 assignments: 35.8 us here against about 15 us).
constexpr int DS_SMALL_MAX = 1024;

// Exclusive scan over the 1024 threads of a block (wave scans, then the wave
// totals in order).  Returns this thread's exclusive prefix; *total gets the sum.
__device__ __forceinline__ int block_exscan_1024(int v, int* wave_tot, int* total) {
    const int lane = lane_id();
    const int wv = threadIdx.x / kWave;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
    }
    if (lane == kWave - 1) wave_tot[wv] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < 1024 / kWave; ++w) {
        if (w < wv) before += wave_tot[w];
        all += wave_tot[w];
    }
    *total = all;
    return before + incl - v;
}

// count + scan + scatter of n <= DS_SMALL_MAX assignments ids[0..n) (global
// or LDS) by a block of 1024 threads (thread e owns expert e in the scan;
// E <= 1024).  hist and offs: 1024 ints of LDS each; wave_tot: 16 ints.
// Integer adds commute, so the LDS histogram is exact; the ranks come from
// ballots in flat order, never from an atomic.  Returns the routed count of
// expert threadIdx.x (0 for threads >= E).
__device__ __forceinline__ int dispatch_small_block(
    int n, int E, int nbits, int capacity, const int32_t* ids, int32_t* __restrict__ counts,
    int32_t* __restrict__ kept, int32_t* __restrict__ offsets, int32_t* __restrict__ assign_row,
    int32_t* __restrict__ row_assign, int* hist, int* offs, int* wave_tot) {
    const int tid = threadIdx.x;
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 1024) {
        const int e = ids[i];
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    const int c = tid < E ? hist[tid] : 0;
    const int kp = tid < E ? (capacity < 0 ? c : min(c, capacity)) : 0;
    int S = 0;
    const int excl = block_exscan_1024(kp, wave_tot, &S);
    if (tid < E) {
        counts[tid] = c;
        kept[tid] = kp;
        offsets[tid] = excl;
        offs[tid] = excl;
    }
    if (tid == 0) offsets[E] = S;
    hist[tid] = 0;  // from here on: running rank per expert
    __syncthreads();
    if (tid < kWave) {
        const int lane = tid;
        const unsigned long long below = (1ull << lane) - 1ull;
        for (int base = 0; base < n; base += kWave) {
            const int i = base + lane;
            const bool in = i < n;
            const int e = in ? ids[i] : -1;
            const bool ok = in && (unsigned)e < (unsigned)E;
            unsigned long long peers = __ballot(ok);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = ok && ((e >> b) & 1);
                const unsigned long long bb = __ballot(bit);
                peers &= bit ? bb : ~bb;
            }
            if (ok) {
                const int r0 = hist[e];
                const int rank = r0 + __popcll(peers & below);
                const int last = 63 - __clzll(peers);
                if (capacity < 0 || rank < capacity) {
                    const int row = offs[e] + rank;
                    assign_row[i] = row;
                    if ((unsigned)row < (unsigned)n) row_assign[row] = i;
                } else {
                    assign_row[i] = -1;
                }
                if (lane == last) hist[e] = r0 + __popcll(peers);
            } else if (in) {
                assign_row[i] = -1;
            }
        }
    }
    // Rows past the kept total S carry no assignment (disjoint from the rows above).
    for (int j = S + tid; j < n; j += 1024) row_assign[j] = -1;
    return c;
}

}  // namespace moe
