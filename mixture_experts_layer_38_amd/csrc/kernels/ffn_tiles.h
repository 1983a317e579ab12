// Pieces of the tiled expert-GEMM kernels (ffn_prefill.hip): the
// XCD-partitioned, expert-grouped tile order, the swizzle of 128-byte LDS tile
// rows, and explicit wait counts.
#pragma once

#include "../device_common.h"

namespace moe {

constexpr int PF_GM = 8;   // row tiles per group in the tile order
constexpr int PF_XCD = 8;  // XCDs: workgroup b runs on XCD b % 8

// Swizzle of the eight 16-byte chunks of a 128-byte tile row: row r keeps
// chunk c in slot c ^ pf_swz(r), so fragment reads of consecutive rows (one
// chunk each) fall in distinct banks.
__device__ __forceinline__ int pf_swz(int r) { return (r ^ (r >> 3)) & 7; }

// s_waitcnt immediate: vmcnt <= n, no wait on the other counters.
#define PF_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | ((((n) >> 4) & 3) << 14))
// s_waitcnt immediate: lgkmcnt == 0, no wait on the other counters.
#define PF_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14))

// v itself, passed through an empty asm statement (no instruction): the
// compiler keeps it after the memory operations issued before it, so a load
// whose value goes through it is waited for only here.
__device__ __forceinline__ int pf_opaque_v(int v) {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+v"(v));
#endif
    return v;
}

// The lane index, computed anew at this point: the compiler cannot reuse an
// earlier copy (which it would keep in a register across the main loop).
__device__ __forceinline__ int pf_lane_fresh() {
    int v = 0;
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
#endif
    return v;
}

// The tiled kernel's per-wave block counts, encoded in one compile-time
// value v: v < PF_HT, 4 weight blocks x v token blocks (32 rows each) per
// wave (the 2 x 2 layout); v = PF_HT + n, the 1 x 4 layout's 2 weight blocks
// x n token blocks, in which a stage loads only the tile's first n token
// blocks (load instruction j fills token rows [32 j, 32 j + 32)).
constexpr int PF_HT = 16;
__host__ __device__ constexpr int pf_tblocks(int v) { return v >= PF_HT ? v - PF_HT : v; }
__host__ __device__ constexpr int pf_wblocks(int v) { return v >= PF_HT ? 2 : 4; }
__host__ __device__ constexpr int pf_aloads(int v, int nja) { return v >= PF_HT ? v - PF_HT : nja; }

// Tile t of the grouped order: row tile mt (of expert e, rows [row0, row_end))
// and weight tile nt.  A group of g row tiles starting at row tile m0 owns
// tiles [m0 n_nt, (m0 + g) n_nt), row tile fastest, so tile t lies in the
// group of row tile t / n_nt.
struct PfTile {
    int mt, nt, e, row0, row_end;
};
__device__ __forceinline__ PfTile pf_tile(int t, int n_mt, int n_nt, const int32_t* mt_expert,
                                          const int32_t* mt_row0, const int32_t* offsets, int n_rows) {
    PfTile r;
    const int m = t / n_nt;
    const int v = mt_expert[m];
    const int gsize = ((v >> 11) & 7) + 1;
    const int first = m - ((v >> 14) & 7);
    const int rem = t - first * n_nt;
    r.mt = first + rem % gsize;
    r.nt = rem / gsize;
    r.e = mt_expert[r.mt] & 0x7FF;
    r.row0 = mt_row0[r.mt];
    r.row_end = min(offsets[r.e + 1], n_rows);
    return r;
}

// Row tiles the plan may produce for n_rows grouped rows over E experts (tiles
// of at least 128 rows, one partial tile per expert).
int prefill_max_mtiles(int n_rows, int E);

}  // namespace moe
