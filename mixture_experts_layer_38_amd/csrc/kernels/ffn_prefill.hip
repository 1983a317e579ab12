// Grouped SwiGLU FFN for large expert groups (prefill): MoE notes
// (www.cf-1.com/news/5905749) §2 step 3 and §2.3 (batched permute, then one
// batched GEMM per expert group); the engineering page
// (ybb.press/quantum-computing/18594) §2.3: prefill is compute-bound, so the
// GEMM throughput is what matters.
//
// Both GEMMs are "rows x weights^T" with both operands contiguous along the
// reduction dimension: act = SiLU(X W1^T) * (X W3^T) and h = act W2^T.
//
// Tiles.  A device-side plan (one tiny kernel) cuts every expert's rows into
// 256-row tiles (128-row tiles when the groups average fewer than 128 rows).
// An output tile is 256 (or 128) token rows x 256 weight rows; for gate/up the
// 256 weight rows are 128 features of W1 and the same 128 of W3, interleaved
// in 32-row blocks so that the SiLU-gate epilogue stays inside each wave.
// Four waves (one per SIMD) split a full tile 2 x 2; a wave owns 128 x 128 as
// 4 x 4 blocks of 32x32 accumulated in AGPRs with v_mfma_f32_32x32x16_bf16
// (weights as the first operand, so that each lane ends with four consecutive
// output columns of one token).  An expert's last, partly filled 256-row tile
// of at most 224 rows is split 1 x 4 instead: each wave owns 64 weight rows
// against the tile's token blocks that hold rows (1 to 7), and only those
// rows are loaded.  In 128-row tiles each wave of a partly filled tile runs a
// copy of the main loop that multiplies only its token blocks holding rows.
//
// Pipeline (K a multiple of 64).  Operand stages are 64 wide in k, so a tile
// row is one 128-byte line, and go straight from HBM/L2 into LDS with
// global_load_lds_dwordx4 (no staging registers).  256-row tiles use all
// 160 KB of the LDS as five 32 KB units that the token and weight halves of
// consecutive stages take in turn, one half issued two stages ahead, the other
// one; 128-row tiles use three whole-stage slots.  One barrier per stage.
// Row r keeps its 16-byte chunk c in slot c ^ swz(r), so the fragment reads
// of consecutive rows are free of bank conflicts (the global addresses carry
// the permutation, since the DMA writes lanes in order).  Inside a stage the
// LDS reads of each 16-wide k quarter are interleaved with the MFMAs of the
// quarter before.  Other K use a generic variant further down.
//
// Order.  Workgroup b runs on XCD b % 8.  The tiles are listed expert by
// expert in groups of at most PF_GM row tiles of one expert (row tile fastest
// inside a group), and XCD x takes the x-th contiguous eighth of that list, so
// the tiles that run together on one XCD share their token rows and weight
// rows in its L2.  In GEMMs of at least 8 rounds per XCD, the last two rounds
// of each XCD's list are claimed at run time (per-XCD counters), so that an
// XCD that runs ahead takes over tiles of one that runs behind.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "../device_common.h"
#include "../launch.h"
#include "ffn_tiles.h"

namespace moe {

constexpr int PF_BN = 256;          // weight rows per tile
constexpr int PF_BK = 64;           // k per pipeline stage (128-byte tile rows)
constexpr int PF_THREADS = 256;
constexpr int PF_BM_MAX = 256;      // token rows per tile: 256, or 128 for small groups
constexpr int PF_SMALL_MIN_E = 32;  // experts from which small groups leave the tiled GEMM

int prefill_max_mtiles(int n_rows, int E) { return n_rows / 128 + E + 1; }

// One block; zeroes the two GEMMs' tail-claim counters (claim, 2 x 8,
// optional), and thread e cuts expert e's rows into bm-row tiles: *mt_count
// row tiles, tile j starting at grouped row mt_row0[j].  mt_expert[j] packs
// the tile's expert (bits 0-10) and its place in the tile order's groups:
// each expert's row tiles form ceil(n / PF_GM) groups of balanced sizes, so
// that no group mixes experts (a group's weight tiles are then shared by all
// of its row tiles); bits 11-13 hold the group's size - 1, bits 14-16 the
// tile's position in it.
__global__ __launch_bounds__(1024) void ffn_plan_kernel(int E, int max_mt, int bm, int min_rows,
                                                       const int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ mt_count,
                                                       int32_t* __restrict__ mt_expert,
                                                       int32_t* __restrict__ mt_row0,
                                                       int32_t* __restrict__ small_count,
                                                       int32_t* __restrict__ small_list,
                                                       int32_t* __restrict__ claim) {
    __shared__ int wave_tot[1024 / kWave];
    __shared__ int small_tot[1024 / kWave];
    const int e = threadIdx.x;
    const int lane = e & (kWave - 1);
    const int wv = e / kWave;
    if (claim != nullptr && e < 2 * PF_XCD) claim[e] = 0;  // the GEMMs' tail-claim counters
    const int rows0 = (e < E) ? offsets[e + 1] - offsets[e] : 0;
    // Experts with 1 .. min_rows rows leave the tiled GEMM when they are at
    // least a quarter of all experts (a skewed routing); otherwise every
    // expert stays in it.  Listed in expert order.
    const int sm0 = (e < E && rows0 > 0 && rows0 <= min_rows) ? 1 : 0;
    const unsigned long long bal = __ballot(sm0);
    if (lane == 0) small_tot[wv] = __popcll(bal);
    __syncthreads();
    int sbefore = 0, sall = 0;
    for (int w = 0; w < 1024 / kWave; ++w) {
        if (w < wv) sbefore += small_tot[w];
        sall += small_tot[w];
    }
    const bool split_small = 4 * sall >= E;
    if (split_small && sm0) small_list[sbefore + __popcll(bal & ((1ull << lane) - 1ull))] = e;
    if (e == 0) *small_count = split_small ? sall : 0;
    const int rows = (split_small && sm0) ? 0 : rows0;
    const int nt = (rows + bm - 1) / bm;
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
    if (e < E && nt > 0) {
        const int ng = (nt + PF_GM - 1) / PF_GM;
        const int base = nt / ng, extra = nt % ng;  // group g: base + (g < extra) tiles
        const int big = extra * (base + 1);
        for (int j = 0; j < nt && start + j < max_mt; ++j) {
            const int g = j < big ? j / (base + 1) : extra + (j - big) / base;
            const int gsz = base + (g < extra ? 1 : 0);
            const int g0 = g * base + min(g, extra);
            mt_expert[start + j] = e | ((gsz - 1) << 11) | ((j - g0) << 14);
            mt_row0[start + j] = offsets[e] + j * bm;
        }
    }
    if (e == E - 1) *mt_count = min(start + nt, max_mt);
}

// Split of the last, partly filled round of tiles.  Each XCD runs its
// per_xcd tiles on cpx compute units in rounds of cpx; when the last round
// holds at most half of cpx tiles, each of those rem tiles is cut into nsplit
// ranges of k (nsplit * rem <= cpx), whose fp32 partial sums a second kernel
// adds in range order.  nsplit = 1: no split.
struct PfSplit {
    int full, rem, nsplit;
};
__host__ __device__ __forceinline__ PfSplit pf_split(int per_xcd, int cpx) {
    PfSplit r{per_xcd, 0, 1};
    if (cpx <= 1) return r;
    const int full = per_xcd / cpx * cpx;
    const int rem = per_xcd - full;
    if (rem > 0 && 2 * rem <= cpx) {
        r.full = full;
        r.rem = rem;
        r.nsplit = min(4, cpx / rem);
    }
    return r;
}
constexpr int PF_MAX_CPX = 32;  // compute units per XCD the split buffer is sized for
// Tail rounds of each XCD's tiles that are claimed at run time, for GEMMs of
// at least PF_DYN_MIN_ROUNDS rounds per XCD.
constexpr int PF_DYN_ROUNDS = 2;
constexpr int PF_DYN_MIN_ROUNDS = 8;

// N: weight rows of one expert (gate/up: F, down: d); K: reduction length,
// a multiple of PF_BK; n_nt: weight tiles per row tile.  BM: token rows per
// tile (256, or 128 for small expert groups); NSLOT: LDS stages in the ring.
// SPLIT = false: every tile except the k-split ones of the last round;
// SPLIT = true: only the k ranges of those (fp32 partial tiles into part).
template <bool GATED, int BM, int NSLOT, bool SPLIT>
__global__ __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ffn_prefill_kernel(
    int n_rows, int N, int K, int n_nt, const bf16* __restrict__ A,
    const int32_t* __restrict__ rowmap, int topk, const int32_t* __restrict__ mt_count, const int32_t* __restrict__ mt_expert,
    const int32_t* __restrict__ mt_row0, const int32_t* __restrict__ offsets,
    const bf16* __restrict__ Wa, const bf16* __restrict__ Wb, bf16* __restrict__ out, int cpx,
    float* __restrict__ part, int32_t* __restrict__ claim, int cus) {
    constexpr int SA = BM * PF_BK;      // bf16 elements of one A stage
    constexpr int SB = PF_BN * PF_BK;   // bf16 elements of one B stage
    constexpr int NTB = BM / 64;        // 32-row token blocks per wave
    constexpr int NJA = BM / 32;        // A load instructions per wave per stage
    constexpr int NJB = PF_BN / 32;     // B load instructions per wave per stage
    constexpr int NLD = NJA + NJB;      // loads per wave per stage
    static_assert(NSLOT == 2 || NSLOT == 3 || (NSLOT == 5 && SA == SB), "slot scheme");
    // NSLOT 2 or 3: that many whole stages (an A and a B slot each).  NSLOT 5:
    // five half-stage units of 32 KB (all 160 KB of the LDS) that the A and B
    // halves of consecutive stages take in turn.
    constexpr bool HALF = NSLOT == 5;
    __shared__ __align__(1024) bf16 sA0[SA], sA1[SA], sA2[NSLOT == 3 ? SA : 1];
    __shared__ __align__(1024) bf16 sB0[SB], sB1[SB], sB2[NSLOT == 3 ? SB : 1];
    __shared__ __align__(1024) bf16 sU4[HALF ? SB : 1];
    const int n_mt = *mt_count;
    const int tiles = n_mt * n_nt;
    const int per_xcd = (tiles + PF_XCD - 1) / PF_XCD;
    const int xcd = blockIdx.x % PF_XCD;
    int slot = blockIdx.x / PF_XCD;
    // The gate/up epilogue is not linear in the sums, so only the second GEMM splits.
    const PfSplit sp = GATED ? PfSplit{per_xcd, 0, 1} : pf_split(per_xcd, cpx);
    int kpart = 0;
    constexpr bool split = SPLIT;
    int t;
    if (SPLIT) {
        const int u = slot;
        if (sp.nsplit <= 1 || u >= sp.rem * sp.nsplit) return;
        slot = sp.full + u / sp.nsplit;
        kpart = u % sp.nsplit;
        if (slot >= per_xcd) return;
        t = xcd * per_xcd + slot;
        if (t >= tiles) return;
    } else {
        // XCD v's main list: its first main(v) tiles (all of them, or those
        // before the split round).  With claim counters, the last
        // min(PF_DYN_ROUNDS * cus, main(v)) of them (the tail) are claimed at
        // run time when the XCDs have at least PF_DYN_MIN_ROUNDS rounds of
        // tiles each (shorter GEMMs lost more to the claims than they gained
        // from the balance): the workgroups of slots [main - tail, main + cus) take
        // the next unclaimed tile of their own XCD's tail, else of another
        // XCD's (in the order xcd + 1, xcd + 2, ...), so that an XCD that
        // runs ahead takes over the tail of one that runs behind; the cus
        // extra workgroups per XCD are the ones that can take over.  Each
        // tile is still computed whole by one workgroup, so the results do
        // not depend on which workgroup claims it.
        auto main_of = [&](int v) {
            const int nv = min(per_xcd, max(0, tiles - v * per_xcd));
            return sp.nsplit > 1 ? min(nv, sp.full) : nv;
        };
        const int dyn = (claim != nullptr && per_xcd >= PF_DYN_MIN_ROUNDS * cus) ? PF_DYN_ROUNDS * cus : 0;
        const int mx = main_of(xcd);
        const int dx = min(dyn, mx);
        if (slot < mx - dx) {
            t = xcd * per_xcd + slot;
        } else {
            if (dyn == 0 || slot >= mx + cus) return;
            int* bc = reinterpret_cast<int*>(sA0);  // broadcast through the first LDS slot
            if (threadIdx.x == 0) {
                int got = -1;
                for (int j = 0; j < PF_XCD && got < 0; ++j) {
                    const int v = (xcd + j) % PF_XCD;
                    const int mv = main_of(v);
                    const int dv = min(dyn, mv);
                    if (dv <= 0) continue;
                    if (j > 0 && __hip_atomic_load(&claim[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= dv)
                        continue;
                    const int i = atomicAdd(&claim[v], 1);
                    if (i < dv) got = v * per_xcd + (mv - dv) + i;
                }
                bc[0] = got;
            }
            __syncthreads();
            t = __builtin_amdgcn_readfirstlane(bc[0]);
            __syncthreads();  // every wave has read it before the loads refill the slot
            if (t < 0) return;
        }
    }
    const PfTile tl = pf_tile(t, n_mt, n_nt, mt_expert, mt_row0, offsets, n_rows);
    const int nt = tl.nt;
    const int e = tl.e;
    const int row0 = tl.row0;
    const int row_end = tl.row_end;
    // k range of this launch unit: all of K, or range kpart of nsplit
    const int nk_all = K / PF_BK;
    const int ks0 = split ? nk_all * kpart / sp.nsplit : 0;
    const int nk = split ? nk_all * (kpart + 1) / sp.nsplit - ks0 : nk_all;

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int lane = lane_id();

    // Loads: a stage is BM/8 A and 32 B wave instructions of 8 rows x 128
    // bytes; wave w issues rows [8 (w + 4 j), +8) of each.  Lane p fills slot
    // p % 8 of tile row p / 8 of its instruction, fetching the chunk that the
    // swizzle puts there.  Tile rows past the expert's last row all read that
    // last row (one line per stage, which the cache merges), so a partly
    // filled tile asks L2 for little more than its real rows; every wave still
    // issues the same number of loads on every stage.
    const int lr = lane >> 3;
    const int ls = lane & 7;
    const bf16* a_src[NJA];
    const bf16* b_src[NJB];
    // Token row of A load j.  Through the row map, all its loads go out at
    // once (a test of the map inside the loop put each behind a wait of its
    // own), before the weights' first loads, and the rows are formed after
    // those (src_row's arithmetic).
    int arow[NJA];
    if (rowmap != nullptr) {
#pragma unroll
        for (int j = 0; j < NJA; ++j) arow[j] = rowmap[min(row0 + 8 * (wave + 4 * j) + lr, row_end - 1)];
    } else {
#pragma unroll
        for (int j = 0; j < NJA; ++j) arow[j] = min(row0 + 8 * (wave + 4 * j) + lr, row_end - 1);
    }
#pragma unroll
    for (int j = 0; j < NJB; ++j) {
        const int tr = 8 * (wave + 4 * j) + lr;
        const int c = ls ^ pf_swz(tr);
        if (GATED) {
            // tile rows [128 w, 128 w + 128) = W1, W3, W1, W3 blocks of 32 rows
            // for features nt*128 + 64 w + [0, 64)
            const int w = tr >> 7;
            const int blk = (tr >> 5) & 3;
            const int f = min(nt * 128 + w * 64 + (blk >> 1) * 32 + (tr & 31), N - 1);
            const bf16* W = (blk & 1) ? Wb : Wa;
            b_src[j] = W + ((size_t)e * N + f) * K + (size_t)ks0 * PF_BK + c * 8;
        } else {
            const int nr = min(nt * PF_BN + tr, N - 1);
            b_src[j] = Wa + ((size_t)e * N + nr) * K + (size_t)ks0 * PF_BK + c * 8;
        }
    }
    // nja: the A loads of a stage (NJA, or the tile's token blocks in the 1 x 4 layout)
    auto issue_a = [&](int kt, bf16* dA, auto nja) __attribute__((always_inline)) {
        const size_t ko = (size_t)min(kt, nk - 1) * PF_BK;
#pragma unroll
        for (int j = 0; j < decltype(nja)::value; ++j)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a_src[j] + ko),
                                             (__attribute__((address_space(3))) void*)(dA + 8 * (wave + 4 * j) * PF_BK),
                                             16, 0, 0);
    };
    auto issue_b = [&](int kt, bf16* dB) __attribute__((always_inline)) {
        const size_t ko = (size_t)min(kt, nk - 1) * PF_BK;
#pragma unroll
        for (int j = 0; j < NJB; ++j)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(b_src[j] + ko),
                                             (__attribute__((address_space(3))) void*)(dB + 8 * (wave + 4 * j) * PF_BK),
                                             16, 0, 0);
    };
    auto issue = [&](int kt, bf16* dA, bf16* dB) __attribute__((always_inline)) {
        issue_a(kt, dA, std::integral_constant<int, NJA>{});
        issue_b(kt, dB);
    };

    const int wm = wave & 1;   // token half of the tile (BM / 2 rows)
    const int wn = wave >> 1;  // weight half of the tile (128 rows)
    // Token blocks of the tile that hold at least one row of the expert.
    const int nhb = __builtin_amdgcn_readfirstlane((row_end - row0 + 31) / 32);
    // 1 x 4 layout (256-row tiles holding at most 224 rows, an expert's last,
    // partly filled tile): in the 2 x 2 layout the waves of the second token
    // half would multiply fewer blocks (or none) and wait at every barrier
    // for those of the first, so instead wave w owns the tile's weight rows
    // [64 w, 64 w + 64) against all nhb token blocks, and only those blocks'
    // rows are loaded.  Every wave then multiplies 8 nhb blocks per stage
    // instead of at most 16.
    const bool ht = HALF && nhb <= 2 * NTB - 1;
    const int wrow0 = ht ? 64 * wave : wn * 128;      // first weight row of the wave's blocks
    const int trow0 = ht ? 0 : wm * (BM / 2);         // first token row of the wave's blocks
    // Through a row map, the weights of stages 0 and 1 are requested before
    // the token rows' addresses exist (those wait for the map), into the units
    // where the main loop expects them; run() then requests the token rows of
    // both stages.  Loads return in order, so once only the last stage's
    // token loads are in flight, the map and stage 0 have arrived.  Without a
    // map, run() requests both stages in the usual order.
    const bool wfirst = rowmap != nullptr;
    if (wfirst) {
        if (HALF && ht) {
            issue_b(0, sA0);
            issue_b(1, sA1);
        } else {
            issue_b(0, sB0);
            issue_b(1, sB1);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NJA; ++j) {
        const int tr = 8 * (wave + 4 * j) + lr;
        // assignment -> token (src_row): a dropped slot (-1) reads token 0
        const int a = pf_opaque_v(arow[j]);  // waited for here, after the weights' loads
        const int r = rowmap != nullptr ? (a < 0 ? 0 : a / topk) : a;
        a_src[j] = A + (size_t)r * K + (size_t)ks0 * PF_BK + (ls ^ pf_swz(tr)) * 8;
    }
    // acc[wb + 2 (tb / 4)][tb % 4]: the accumulators of weight block wb and
    // token block tb (4 x NTB blocks in the 2 x 2 layout, 2 x 2 NTB in 1 x 4).
    f32x16 acc[4][NTB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NTB; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    // Fragment rows: weight rows wrow0 + 32 wb + lane%32, token rows
    // trow0 + 32 tb + lane%32; their swizzles are fixed for the whole tile.
    const int fhalf = lane >> 5;
    int wsw[4], tsw[2 * NTB];
#pragma unroll
    for (int i = 0; i < 4; ++i) wsw[i] = pf_swz(wrow0 + i * 32 + (lane & 31));
#pragma unroll
    for (int i = 0; i < 2 * NTB; ++i) tsw[i] = pf_swz(trow0 + i * 32 + (lane & 31));
    struct Frags {
        bf16x8 w[4], t[2 * NTB];
    };
    // 16-wide k quarter q of a stage: chunk 2q + (lane / 32).  nb encodes the
    // wave's blocks: nb < PF_HT, 4 weight blocks x nb token blocks (NTB, or
    // fewer on a partly filled tile whose last blocks hold only padded rows);
    // nb = PF_HT + n, the 1 x 4 layout's 2 weight blocks x n token blocks.
    auto read = [&](auto nb, const bf16* cA, const bf16* cB, int q, Frags& f) __attribute__((always_inline)) {
        constexpr int NB = pf_tblocks(decltype(nb)::value), WB = pf_wblocks(decltype(nb)::value);
        const int c = 2 * q + fhalf;
#pragma unroll
        for (int wb = 0; wb < WB; ++wb)
            f.w[wb] = *reinterpret_cast<const bf16x8*>(
                &cB[(wrow0 + wb * 32 + (lane & 31)) * PF_BK + (c ^ wsw[wb]) * 8]);
#pragma unroll
        for (int tb = 0; tb < NB; ++tb)
            f.t[tb] = *reinterpret_cast<const bf16x8*>(
                &cA[(trow0 + tb * 32 + (lane & 31)) * PF_BK + (c ^ tsw[tb]) * 8]);
    };
    auto mma = [&](auto nb, const Frags& f) __attribute__((always_inline)) {
        constexpr int NB = pf_tblocks(decltype(nb)::value), WB = pf_wblocks(decltype(nb)::value);
#pragma unroll
        for (int wb = 0; wb < WB; ++wb)
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                f32x16& a = acc[wb + 2 * (tb >> 2)][tb & 3];
                a = mfma32(f.w[wb], f.t[tb], a);
            }
    };
    // Interleave: one MFMA, then one LDS fragment read, for every read of the
    // next quarter, then the remaining MFMAs (the reads issue in the shadow of
    // the MFMAs); NV loads (at most one per MFMA) are spread evenly over the
    // quarter's MFMAs.
    auto interleave = [&](auto nb, auto nv_c) __attribute__((always_inline)) {
        constexpr int NV = decltype(nv_c)::value;
        constexpr int NB = pf_tblocks(decltype(nb)::value), WB = pf_wblocks(decltype(nb)::value);
        constexpr int NM = WB * NB;
        constexpr int DM = NM > 0 ? NM : 1;  // a wave with no blocks has no MFMAs to spread over
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < WB + NB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            const int nl = ((i + 1) * NV) / DM - (i * NV) / DM;  // loads after MFMA i
#pragma unroll
            for (int l = 0; l < (NV + DM - 1) / DM; ++l)
                if (l < nl) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
    };
    // After the barrier: the last quarter's MFMAs, NV loads and the reads of
    // the next stage's first quarter, one of each in turn, so no wave stalls
    // on a burst of loads with its MFMAs waiting.
    auto interleave_loads = [&](auto nb, auto nv_c) __attribute__((always_inline)) {
        constexpr int NV = decltype(nv_c)::value;
        constexpr int NB = pf_tblocks(decltype(nb)::value), WB = pf_wblocks(decltype(nb)::value);
        constexpr int NM = WB * NB, NR = WB + NB;
        constexpr int NI = NM > NV ? NM : NV;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            if (i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            if (i < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };
    // Stage kt is multiplied in four 16-wide quarters; the LDS reads of each
    // quarter overlap the MFMAs of the quarter before.  After the third
    // quarter's MFMAs: wait until this wave's reads of stage kt are done and
    // its loads of stage kt + 1 have landed (later loads may still be in
    // flight); a barrier then makes stage kt + 1 visible to every wave and
    // tells every wave that stage kt's slots are free.  The reads of the first
    // quarter of stage kt + 1 and the new loads are spread over the last
    // quarter's MFMAs.
    //   NSLOT 2, 3: stage kt is in slot kt % NSLOT; stage kt + NSLOT is
    //     loaded into it right after the barrier.
    //   NSLOT 5: A(kt) is in unit 2 kt % 5, B(kt) in unit (2 kt + 1) % 5.
    //     After the barrier of stage kt, B(kt + 2) is loaded into A(kt)'s unit;
    //     A(kt + 3) goes into B(kt)'s unit during the first three quarters of
    //     stage kt + 1, so the loads of a stage never come in one burst, and
    //     when stage kt ends only A(kt + 2) may still be in flight.
    // Every step issues the same loads and reads (clamped to the last stage
    // at the end, into slots no later step reads), so the counts of loads in
    // flight are the same on every path.
    Frags fa, fb;
    using IC0 = std::integral_constant<int, 0>;
    auto step = [&](auto nb, int kt, bf16* cA, bf16* cB, const bf16* nA, const bf16* nB) __attribute__((always_inline)) {
        read(nb, cA, cB, 1, fb);
        mma(nb, fa);
        interleave(nb, IC0{});
        __builtin_amdgcn_sched_barrier(0);
        read(nb, cA, cB, 2, fa);
        mma(nb, fb);
        interleave(nb, IC0{});
        __builtin_amdgcn_sched_barrier(0);
        read(nb, cA, cB, 3, fb);
        mma(nb, fa);
        interleave(nb, IC0{});
        __builtin_amdgcn_sched_barrier(0);
        PF_WAIT_LGKM0();
        PF_WAIT_VM(NLD * (NSLOT - 2));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue(kt + NSLOT, cA, cB);
        read(nb, nA, nB, 0, fa);
        mma(nb, fb);
        interleave_loads(nb, std::integral_constant<int, NLD>{});
        __builtin_amdgcn_sched_barrier(0);
    };
    // pA: the unit that receives A(kt + 2) during this step.
    //   1 x 4 layout: the token rows (at most 224 of a stage, mostly L2
    //     hits) and the weights (a whole stage, streamed from HBM) trade
    //     places: the weights of stage kt + 2 take the early loads into the
    //     "A" unit, the token rows the loads after the barrier into the other,
    //     so the weights get two stages of lead.  The units' roles swap with
    //     them (SW below).
    auto step5 = [&](auto nb, int kt, bf16* cA, bf16* cB, const bf16* nA, const bf16* nB, bf16* pA) __attribute__((always_inline)) {
        constexpr bool SW = pf_wblocks(decltype(nb)::value) == 2;
        constexpr int NJ = pf_aloads(decltype(nb)::value, NJA);  // A loads of a stage
        constexpr int NE = SW ? NJB : NJ;  // early loads, spread over the first three quarters
        constexpr int NL = SW ? NJ : NJB;  // loads after the barrier
        constexpr int V0 = (NE + 2) / 3, V1 = (NE + 1) / 3, V2 = NE / 3;
        static_assert(V0 + V1 + V2 == NE, "early loads per quarter");
        const size_t ko = (size_t)min(kt + 2, nk - 1) * PF_BK;
        auto ld = [&](int j) __attribute__((always_inline)) {
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)((SW ? b_src[j] : a_src[j]) + ko),
                                             (__attribute__((address_space(3))) void*)(pA + 8 * (wave + 4 * j) * PF_BK),
                                             16, 0, 0);
        };
        // this stage's token rows and weights, and the next stage's
        const bf16* tA = SW ? cB : cA;
        const bf16* tB = SW ? cA : cB;
        const bf16* uA = SW ? nB : nA;
        const bf16* uB = SW ? nA : nB;
        read(nb, tA, tB, 1, fb);
#pragma unroll
        for (int j = 0; j < V0; ++j) ld(j);
        mma(nb, fa);
        interleave(nb, std::integral_constant<int, V0>{});
        __builtin_amdgcn_sched_barrier(0);
        read(nb, tA, tB, 2, fa);
#pragma unroll
        for (int j = V0; j < V0 + V1; ++j) ld(j);
        mma(nb, fb);
        interleave(nb, std::integral_constant<int, V1>{});
        __builtin_amdgcn_sched_barrier(0);
        read(nb, tA, tB, 3, fb);
#pragma unroll
        for (int j = V0 + V1; j < NE; ++j) ld(j);
        mma(nb, fa);
        interleave(nb, std::integral_constant<int, V2>{});
        __builtin_amdgcn_sched_barrier(0);
        PF_WAIT_LGKM0();
        PF_WAIT_VM(NE);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SW)
            issue_a(kt + 2, cA, std::integral_constant<int, NJ>{});
        else
            issue_b(kt + 2, cA);
        read(nb, uA, uB, 0, fa);
        mma(nb, fb);
        interleave_loads(nb, std::integral_constant<int, NL>{});
        __builtin_amdgcn_sched_barrier(0);
    };
    // NSLOT 3: stage kt + 2 goes into slot (kt + 2) % 3, freed when stage
    // kt - 1 ended, with its loads spread over all four quarters of stage kt
    // (it is needed when stage kt + 1 ends); when stage kt ends only the
    // loads issued in its first three quarters may still be in flight.
    auto step3 = [&](auto nb, int kt, bf16* cA, bf16* cB, const bf16* nA, const bf16* nB, bf16* pA, bf16* pB) __attribute__((always_inline)) {
        constexpr int V = (NLD + 3) / 4;
        constexpr int V0 = V, V1 = V, V2 = V, V3 = NLD - 3 * V;
        static_assert(V3 >= 0, "loads per quarter");
        const size_t ko = (size_t)min(kt + 2, nk - 1) * PF_BK;
        auto ld = [&](int i) __attribute__((always_inline)) {
            if (i < NJA)
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(a_src[i] + ko),
                                                 (__attribute__((address_space(3))) void*)(pA + 8 * (wave + 4 * i) * PF_BK),
                                                 16, 0, 0);
            else
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(b_src[i - NJA] + ko),
                                                 (__attribute__((address_space(3))) void*)(pB + 8 * (wave + 4 * (i - NJA)) * PF_BK),
                                                 16, 0, 0);
        };
        read(nb, cA, cB, 1, fb);
#pragma unroll
        for (int i = 0; i < V0; ++i) ld(i);
        mma(nb, fa);
        interleave(nb, std::integral_constant<int, V0>{});
        __builtin_amdgcn_sched_barrier(0);
        read(nb, cA, cB, 2, fa);
#pragma unroll
        for (int i = V0; i < V0 + V1; ++i) ld(i);
        mma(nb, fb);
        interleave(nb, std::integral_constant<int, V1>{});
        __builtin_amdgcn_sched_barrier(0);
        read(nb, cA, cB, 3, fb);
#pragma unroll
        for (int i = V0 + V1; i < V0 + V1 + V2; ++i) ld(i);
        mma(nb, fa);
        interleave(nb, std::integral_constant<int, V2>{});
        __builtin_amdgcn_sched_barrier(0);
        PF_WAIT_LGKM0();
        PF_WAIT_VM(V0 + V1 + V2);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = V0 + V1 + V2; i < NLD; ++i) ld(i);
        read(nb, nA, nB, 0, fa);
        mma(nb, fb);
        interleave_loads(nb, std::integral_constant<int, V3>{});
        __builtin_amdgcn_sched_barrier(0);
    };
    // The main loop for a wave that multiplies nb token blocks.  Every
    // instance issues the same loads and barriers, so the waves of one
    // workgroup may run different instances.
    auto run = [&](auto nb) __attribute__((always_inline)) {
        if constexpr (HALF) {
            bf16* const u0 = sA0;
            bf16* const u1 = sB0;
            bf16* const u2 = sA1;
            bf16* const u3 = sB1;
            bf16* const u4 = sU4;
            constexpr int NJ = pf_aloads(decltype(nb)::value, NJA);
            constexpr bool SW = pf_wblocks(decltype(nb)::value) == 2;  // 1 x 4 layout: roles swapped
            // stage s: B in unit 2s + SW, A in unit 2s + 1 - SW
            if (wfirst) {  // B already requested
                if constexpr (SW) {
                    issue_a(0, u1, std::integral_constant<int, NJ>{});
                    issue_a(1, u3, std::integral_constant<int, NJ>{});
                } else {
                    issue_a(0, u0, std::integral_constant<int, NJ>{});
                    issue_a(1, u2, std::integral_constant<int, NJ>{});
                }
                PF_WAIT_VM(NJ);
            } else {
                if constexpr (SW) {
                    issue_b(0, u0);
                    issue_a(0, u1, std::integral_constant<int, NJ>{});
                    issue_b(1, u2);
                    issue_a(1, u3, std::integral_constant<int, NJ>{});
                } else {
                    issue_a(0, u0, std::integral_constant<int, NJ>{});
                    issue_b(0, u1);
                    issue_a(1, u2, std::integral_constant<int, NJ>{});
                    issue_b(1, u3);
                }
                PF_WAIT_VM(NJ + NJB);
            }
            __builtin_amdgcn_s_barrier();
            if constexpr (SW)
                read(nb, u1, u0, 0, fa);
            else
                read(nb, u0, u1, 0, fa);
            const int nk_main = nk - nk % 5;
            for (int k0 = 0; k0 < nk_main; k0 += 5) {
                step5(nb, k0, u0, u1, u2, u3, u4);
                step5(nb, k0 + 1, u2, u3, u4, u0, u1);
                step5(nb, k0 + 2, u4, u0, u1, u2, u3);
                step5(nb, k0 + 3, u1, u2, u3, u4, u0);
                step5(nb, k0 + 4, u3, u4, u0, u1, u2);
            }
            // The last nk % 5 stages start again at unit 0.
            const int rem = nk - nk_main;
            if (rem > 0) step5(nb, nk_main, u0, u1, u2, u3, u4);
            if (rem > 1) step5(nb, nk_main + 1, u2, u3, u4, u0, u1);
            if (rem > 2) step5(nb, nk_main + 2, u4, u0, u1, u2, u3);
            if (rem > 3) step5(nb, nk_main + 3, u1, u2, u3, u4, u0);
        } else if constexpr (NSLOT == 3) {
            if (wfirst) {
                issue_a(0, sA0, std::integral_constant<int, NJA>{});
                issue_a(1, sA1, std::integral_constant<int, NJA>{});
                PF_WAIT_VM(NJA);
            } else {
                issue(0, sA0, sB0);
                issue(1, sA1, sB1);
                PF_WAIT_VM(NLD);
            }
            __builtin_amdgcn_s_barrier();
            read(nb, sA0, sB0, 0, fa);
            const int nk_main = nk - nk % 3;
            for (int k0 = 0; k0 < nk_main; k0 += 3) {
                step3(nb, k0, sA0, sB0, sA1, sB1, sA2, sB2);
                step3(nb, k0 + 1, sA1, sB1, sA2, sB2, sA0, sB0);
                step3(nb, k0 + 2, sA2, sB2, sA0, sB0, sA1, sB1);
            }
            // The last nk % 3 stages start again at slot 0.
            if (nk - nk_main > 0) step3(nb, nk_main, sA0, sB0, sA1, sB1, sA2, sB2);
            if (nk - nk_main > 1) step3(nb, nk_main + 1, sA1, sB1, sA2, sB2, sA0, sB0);
        } else {
            if (wfirst) {
                issue_a(0, sA0, std::integral_constant<int, NJA>{});
                issue_a(1, sA1, std::integral_constant<int, NJA>{});
                PF_WAIT_VM(NJA);
            } else {
                issue(0, sA0, sB0);
                issue(1, sA1, sB1);
                PF_WAIT_VM(NLD);
            }
            __builtin_amdgcn_s_barrier();
            read(nb, sA0, sB0, 0, fa);
            const int nk_main = nk - nk % 2;
            for (int k0 = 0; k0 < nk_main; k0 += 2) {
                step(nb, k0, sA0, sB0, sA1, sB1);
                step(nb, k0 + 1, sA1, sB1, sA0, sB0);
            }
            if (nk - nk_main > 0) step(nb, nk_main, sA0, sB0, sA1, sB1);
        }
    };
    // 1 x 4 layout: the tile's nhb token blocks, 1 .. 7.  2 x 2 layout: the
    // token blocks of this wave that hold at least one row of the expert
    // (all of them in the 256-row tiles, which use it only from 225 rows on;
    // in 128-row tiles, all of them except on an expert's last, partly
    // filled tile).
    {
        using std::integral_constant;
        const int vh = min(max(row_end - row0 - wm * (BM / 2), 0), BM / 2);
        const int nvb = __builtin_amdgcn_readfirstlane((vh + 31) / 32);
        if constexpr (HALF) {
            static_assert(NTB == 4, "the 1 x 4 layout splits a 256-row tile");
            if (!ht)
                run(integral_constant<int, NTB>{});
            else if (nhb == 1)
                run(integral_constant<int, PF_HT + 1>{});
            else if (nhb == 2)
                run(integral_constant<int, PF_HT + 2>{});
            else if (nhb == 3)
                run(integral_constant<int, PF_HT + 3>{});
            else if (nhb == 4)
                run(integral_constant<int, PF_HT + 4>{});
            else if (nhb == 5)
                run(integral_constant<int, PF_HT + 5>{});
            else if (nhb == 6)
                run(integral_constant<int, PF_HT + 6>{});
            else
                run(integral_constant<int, PF_HT + 7>{});
        } else if (nvb == 0) {
            run(integral_constant<int, 0>{});
        } else if (nvb == 1) {
            run(integral_constant<int, 1>{});
        } else if constexpr (NTB > 3) {
            if (nvb == 2)
                run(integral_constant<int, 2>{});
            else if (nvb == 3)
                run(integral_constant<int, 3>{});
            else
                run(integral_constant<int, NTB>{});
        } else {
            run(integral_constant<int, NTB>{});
        }
    }
    PF_WAIT_VM(0);
    PF_WAIT_LGKM0();

    // Block (wb, tb), acc[wb + 2 (tb / 4)][tb % 4], element i: tile weight
    // row wrow0 + 32 wb + 8*(i/4) + 4*(lane/32) + i%4, tile token row
    // trow0 + 32 tb + lane % 32; the wave holds wbn weight blocks x tbn token
    // blocks (4 x NTB, or 2 x 2 NTB in the 1 x 4 layout).
    const int wbn = ht ? 2 : 4;
    const int tbn = ht ? 2 * NTB : NTB;
    // the lane index again, rather than a value kept across the main loop
    const int el = pf_lane_fresh();
    constexpr int TBMAX = HALF ? 2 * NTB : NTB;  // token blocks of either layout
    // The output through the LDS: each wave puts its block of the tile (token
    // rows trow0 + [0, 32 TBN), the W columns of its weight blocks) into an
    // LDS unit of its own, rows whose 16-byte chunks are swizzled by row, then
    // writes whole row segments, 16 bytes per lane (16 bytes per lane straight
    // from the accumulators would split every row into 16-byte pieces, one
    // request each, 32 rows per instruction).  The barrier makes sure no wave
    // still reads the ring.
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    bf16* const st = wave == 0 ? (NSLOT == 5 ? sA0 : sB0)
                   : wave == 1 ? (NSLOT == 5 ? sB0 : sB1)
                   : wave == 2 ? (NSLOT == 5 ? sA1 : (NSLOT == 3 ? sB2 : sA1))
                               : (NSLOT == 5 ? sB1 : sA0);
    constexpr int UNIT = (NSLOT == 5 ? SB : SA) * (int)sizeof(bf16);  // bytes of the smallest unit used
    // SPLIT: the fp32 partial tile [BM][PF_BN] (row = token, column = weight
    // row) of this k range, in passes of rows that fit the unit.
    auto store_part = [&](auto wbn_c, auto tbn_c) __attribute__((always_inline)) {
        constexpr int WBN = decltype(wbn_c)::value, TBN = decltype(tbn_c)::value;
        constexpr int W = 32 * WBN;                 // fp32 columns of the wave's block
        constexpr int NCH = W / 4;                  // 16-byte chunks per row
        constexpr int RP = UNIT / (W * 4);          // rows per pass
        constexpr int RPI = kWave / NCH;            // rows per store instruction
        static_assert(RP % 32 == 0 && (TBN * 32) % RP == 0, "whole token blocks per pass");
        float* const sf = reinterpret_cast<float*>(st);
        float* pt = part + (size_t)((xcd * sp.rem + (slot - sp.full)) * sp.nsplit + kpart) * BM * PF_BN;
#pragma unroll
        for (int pass = 0; pass < TBN * 32 / RP; ++pass) {
#pragma unroll
            for (int tb = pass * RP / 32; tb < (pass + 1) * RP / 32; ++tb) {
                if (tb >= tbn) continue;
                const int rl = tb * 32 + (el & 31) - pass * RP;
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int wb = 0; wb < WBN; ++wb) {
                        const f32x16& a = acc[wb + 2 * (tb >> 2)][tb & 3];
                        const int cl = wb * 32 + 8 * q + 4 * (el >> 5);
                        *reinterpret_cast<f32x4*>(sf + rl * W + (((cl >> 2) ^ (rl & 7)) << 2)) =
                            f32x4{a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                    }
            }
            const int lrow = el / NCH, lch = el % NCH;
#pragma unroll
            for (int i = 0; i < RP / RPI; ++i) {
                const int rl = i * RPI + lrow;
                const f32x4 v = *reinterpret_cast<const f32x4*>(sf + rl * W + ((lch ^ (rl & 7)) << 2));
                *reinterpret_cast<f32x4*>(pt + (size_t)(trow0 + pass * RP + rl) * PF_BN + wrow0 + lch * 4) = v;
            }
        }
    };
    auto store_tile = [&](auto wbn_c, auto tbn_c) __attribute__((always_inline)) {
        constexpr int WBN = decltype(wbn_c)::value, TBN = decltype(tbn_c)::value;
        constexpr int W = (GATED ? 16 : 32) * WBN;  // bf16 columns of the wave's block
        constexpr int NCH = W / 8;                   // 16-byte chunks per row
        constexpr int SWM = NCH < 8 ? NCH - 1 : 7;   // chunk swizzle: chunk ^ (row & SWM)
        constexpr int RPI = kWave / NCH;             // rows per store instruction
        // a wave's block fits its unit (the ring's 32 KB units; else the
        // smallest slot used, an A slot)
        static_assert(TBN * 32 * W * (int)sizeof(bf16) <= UNIT, "a wave's block fits its LDS unit");
#pragma unroll
        for (int tb = 0; tb < TBN; ++tb) {
            if (tb >= tbn) continue;
            const int rl = tb * 32 + (el & 31);
            bf16* srow = st + rl * W;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int wr = 8 * q + 4 * (el >> 5);
                if constexpr (GATED) {
#pragma unroll
                    for (int pr = 0; pr < WBN / 2; ++pr) {
                        // the wave's weight rows interleave W1 and W3 in
                        // 32-row blocks: local features pr*32 + wr + [0, 4)
                        float v[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            v[r] = silu(acc[2 * pr + 2 * (tb >> 2)][tb & 3][4 * q + r]) *
                                   acc[2 * pr + 1 + 2 * (tb >> 2)][tb & 3][4 * q + r];
                        const int cl = pr * 32 + wr;
                        *reinterpret_cast<bf16x4*>(srow + (((cl >> 3) ^ (rl & SWM)) << 3) + (cl & 7)) =
                            bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
                    }
                } else {
#pragma unroll
                    for (int wb = 0; wb < WBN; ++wb) {
                        const f32x16& av = acc[wb + 2 * (tb >> 2)][tb & 3];
                        const int cl = wb * 32 + wr;
                        *reinterpret_cast<bf16x4*>(srow + (((cl >> 3) ^ (rl & SWM)) << 3) + (cl & 7)) =
                            bf16x4{(bf16)av[4 * q], (bf16)av[4 * q + 1], (bf16)av[4 * q + 2], (bf16)av[4 * q + 3]};
                    }
                }
            }
        }
        // columns of the wave's block in the output: features nt*128 +
        // wrow0 / 2 (gate/up), or weight rows nt*256 + wrow0 (N a multiple of 8)
        const int colbase = GATED ? nt * 128 + wrow0 / 2 : nt * PF_BN + wrow0;
        const int lrow = el / NCH, lch = el % NCH;
        const int gcol = colbase + lch * 8;
#pragma unroll
        for (int i = 0; i < TBN * 32 / RPI; ++i) {
            const int rl = i * RPI + lrow;
            const int grow = row0 + trow0 + rl;
            const bf16x8 val = *reinterpret_cast<const bf16x8*>(st + rl * W + ((lch ^ (rl & SWM)) << 3));
            if (grow < row_end && gcol < N) *reinterpret_cast<bf16x8*>(out + (size_t)grow * N + gcol) = val;
        }
    };
    auto store = [&](auto wbn_c, auto tbn_c) __attribute__((always_inline)) {
        if constexpr (SPLIT)
            store_part(wbn_c, tbn_c);
        else
            store_tile(wbn_c, tbn_c);
    };
    if constexpr (HALF) {
        if (ht)
            store(std::integral_constant<int, 2>{}, std::integral_constant<int, 2 * NTB>{});
        else
            store(std::integral_constant<int, 4>{}, std::integral_constant<int, NTB>{});
    } else {
        store(std::integral_constant<int, 4>{}, std::integral_constant<int, NTB>{});
    }
}

// ---- generic variant (any K) ---------------------------------------------------
constexpr int PG_BM = 256;
constexpr int PG_BN = 256;
constexpr int PG_BK = 64;
constexpr int PG_LDS = PG_BK + 8;  // padded LDS row (bf16 elements)
constexpr int PG_THREADS = 512;
constexpr int PG_XCD = PF_XCD;
constexpr size_t PG_TILE_ELEMS = (size_t)PG_BM * PG_LDS;
constexpr size_t PG_LDS_BYTES = 4 * PG_TILE_ELEMS * sizeof(bf16);

// Generic variant for any K (a multiple of 8): the same tiles, with operands
// staged HBM/L2 -> registers -> LDS (rows padded to 144 bytes), double
// buffered with one 64-wide k step in flight.  N, K, n_nt as above.
template <bool GATED>
__global__ __launch_bounds__(PG_THREADS) void ffn_prefill_generic_kernel(
    int n_rows, int N, int K, int n_nt, const bf16* __restrict__ A,
    const int32_t* __restrict__ rowmap, int topk, const int32_t* __restrict__ mt_count,
    const int32_t* __restrict__ mt_expert, const int32_t* __restrict__ mt_row0,
    const int32_t* __restrict__ offsets, const bf16* __restrict__ Wa, const bf16* __restrict__ Wb,
    bf16* __restrict__ out) {
    extern __shared__ __align__(16) bf16 smem[];
    const int n_mt = *mt_count;
    const int tiles = n_mt * n_nt;
    const int per_xcd = (tiles + PG_XCD - 1) / PG_XCD;
    const int slot = blockIdx.x / PG_XCD;
    if (slot >= per_xcd) return;
    const int t = (blockIdx.x % PG_XCD) * per_xcd + slot;
    if (t >= tiles) return;
    const PfTile tl = pf_tile(t, n_mt, n_nt, mt_expert, mt_row0, offsets, n_rows);
    const int nt = tl.nt;
    const int e = tl.e;
    const int row0 = tl.row0;
    const int row_end = tl.row_end;

    bf16* sA = smem;                      // [2][PG_BM][PG_LDS]
    bf16* sB = smem + 2 * PG_TILE_ELEMS;  // [2][PG_BN][PG_LDS]

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int lane = tid & (kWave - 1);
    const int lr = tid >> 3;        // 0..63: row within a 64-row slab
    const int lc = (tid & 7) * 8;   // 16-byte chunk within the 64-wide k step

    const bf16* a_src[4];
    const bf16* b_src[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = src_row(rowmap, topk, min(row0 + lr + 64 * j, row_end - 1));
        a_src[j] = A + (size_t)r * K + lc;
        const int br = lr + 64 * j;  // weight row inside the tile
        if (GATED) {
            // tile rows [128 w, 128 w + 128) = W1, W3, W1, W3 blocks of 32 rows
            // for features nt*128 + 64 w + [0, 64)
            const int w = br >> 7;
            const int blk = (br >> 5) & 3;
            const int f = min(nt * 128 + w * 64 + (blk >> 1) * 32 + (br & 31), N - 1);
            const bf16* W = (blk & 1) ? Wb : Wa;
            b_src[j] = W + ((size_t)e * N + f) * K + lc;
        } else {
            const int nr = min(nt * PG_BN + br, N - 1);
            b_src[j] = Wa + ((size_t)e * N + nr) * K + lc;
        }
    }

    const int nk = (K + PG_BK - 1) / PG_BK;
    u32x4 ra[4], rb[4];
    auto gload = [&](int kt) {
        const bool ok = kt * PG_BK + lc < K;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ra[j] = load16_or_zero(a_src[j] + (size_t)kt * PG_BK, ok);
            rb[j] = load16_or_zero(b_src[j] + (size_t)kt * PG_BK, ok);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            store16(&sA[buf * PG_TILE_ELEMS + (lr + 64 * j) * PG_LDS + lc], ra[j]);
            store16(&sB[buf * PG_TILE_ELEMS + (lr + 64 * j) * PG_LDS + lc], rb[j]);
        }
    };

    const int wm = wave & 3;   // token block of 64
    const int wn = wave >> 2;  // weight block of 128
    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const bf16* cA = sA + cur * PG_TILE_ELEMS;
        const bf16* cB = sB + cur * PG_TILE_ELEMS;
#pragma unroll
        for (int ks = 0; ks < PG_BK; ks += 16) {
            bf16x8 fw[4], ft[2];
#pragma unroll
            for (int wb = 0; wb < 4; ++wb)
                fw[wb] = *reinterpret_cast<const bf16x8*>(
                    &cB[(wn * 128 + wb * 32 + frag_row) * PG_LDS + ks + frag_k]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
                ft[tb] = *reinterpret_cast<const bf16x8*>(
                    &cA[(wm * 64 + tb * 32 + frag_row) * PG_LDS + ks + frag_k]);
#pragma unroll
            for (int wb = 0; wb < 4; ++wb)
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) acc[wb][tb] = mfma32(fw[wb], ft[tb], acc[wb][tb]);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // acc[wb][tb][i]: weight row 8*(i/4) + 4*(lane/32) + i%4 of block wb,
    // token lane % 32 of block tb.
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int grow = row0 + wm * 64 + tb * 32 + (lane & 31);
        if (grow >= row_end) continue;
        bf16* orow = out + (size_t)grow * N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int wr = 8 * q + 4 * (lane >> 5);
            if (GATED) {
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int f = nt * 128 + wn * 64 + pr * 32 + wr;
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        v[r] = silu(acc[2 * pr][tb][4 * q + r]) * acc[2 * pr + 1][tb][4 * q + r];
                    if (f + 3 < N) {
                        bf16x4 pk = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
                        *reinterpret_cast<bf16x4*>(orow + f) = pk;
                    } else {
                        for (int r = 0; r < 4; ++r)
                            if (f + r < N) orow[f + r] = (bf16)v[r];
                    }
                }
            } else {
#pragma unroll
                for (int wb = 0; wb < 4; ++wb) {
                    const int c = nt * PG_BN + wn * 128 + wb * 32 + wr;
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

// Adds the nsplit partial tiles of each split tile in range order and writes
// the bf16 rows of the second GEMM.  Workgroup (b, y): split tile b / 8 of XCD
// b % 8, rows [16 y, 16 y + 16) of it; every thread issues all its loads at
// once (PF_RD_V float4 of each partial tile).
constexpr int PF_RD_ROWS = 16;
constexpr int PF_RD_V = PF_RD_ROWS * PF_BN / 4 / 256;
template <int BM>
__global__ __launch_bounds__(256) void ffn_split_reduce_kernel(
    int n_rows, int N, int n_nt, int cpx, const int32_t* __restrict__ mt_count,
    const int32_t* __restrict__ mt_expert, const int32_t* __restrict__ mt_row0,
    const int32_t* __restrict__ offsets, const float* __restrict__ part, bf16* __restrict__ out) {
    const int n_mt = *mt_count;
    const int tiles = n_mt * n_nt;
    const int per_xcd = (tiles + PF_XCD - 1) / PF_XCD;
    const PfSplit sp = pf_split(per_xcd, cpx);
    const int xcd = blockIdx.x % PF_XCD;
    const int r = blockIdx.x / PF_XCD;
    if (sp.nsplit <= 1 || r >= sp.rem) return;
    const int t = xcd * per_xcd + sp.full + r;
    if (t >= tiles) return;
    const PfTile tl = pf_tile(t, n_mt, n_nt, mt_expert, mt_row0, offsets, n_rows);
    const int rb = blockIdx.y * PF_RD_ROWS;
    if (tl.row0 + rb >= tl.row_end) return;
    const size_t tsz = (size_t)BM * PF_BN;
    const float* p0 = part + (size_t)((xcd * sp.rem + r) * sp.nsplit) * tsz + (size_t)rb * PF_BN;
    f32x4 v[PF_RD_V];
#pragma unroll
    for (int u = 0; u < PF_RD_V; ++u) v[u] = *reinterpret_cast<const f32x4*>(p0 + (u * 256 + threadIdx.x) * 4);
    for (int p = 1; p < sp.nsplit; ++p)
#pragma unroll
        for (int u = 0; u < PF_RD_V; ++u)
            v[u] += *reinterpret_cast<const f32x4*>(p0 + p * tsz + (u * 256 + threadIdx.x) * 4);
#pragma unroll
    for (int u = 0; u < PF_RD_V; ++u) {
        const int i = (u * 256 + threadIdx.x) * 4;
        const int grow = tl.row0 + rb + i / PF_BN;
        const int gcol = tl.nt * PF_BN + i % PF_BN;
        if (grow >= tl.row_end || gcol >= N) continue;
        bf16* o = out + (size_t)grow * N + gcol;
        if (gcol + 3 < N) {
            *reinterpret_cast<bf16x4*>(o) = bf16x4{(bf16)v[u][0], (bf16)v[u][1], (bf16)v[u][2], (bf16)v[u][3]};
        } else {
            for (int q = 0; q < 4; ++q)
                if (gcol + q < N) o[q] = (bf16)v[u][q];
        }
    }
}

// Compute units per XCD (0: no split), from the current device.
static int prefill_cpx() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (cus % PF_XCD != 0) return 0;
    return min(cus / PF_XCD, PF_MAX_CPX);
}

// Partial tiles of the split: at most PF_MAX_CPX per XCD, and at most four
// per tile of the second GEMM.
static size_t prefill_split_bytes(int n_rows, int E, int d) {
    const size_t parts = std::min((size_t)PF_XCD * PF_MAX_CPX,
                                  (size_t)4 * prefill_max_mtiles(n_rows, E) * ((d + PF_BN - 1) / PF_BN));
    return align_up(parts * PF_BM_MAX * PF_BN * sizeof(float), 256);
}

// Plan: [mt_count][mt_expert][mt_row0][small_count][small_list (E)][claim (2 x 8)].
static size_t prefill_plan_bytes(int n_rows, int E) {
    return align_up((size_t)(2 + 2 * prefill_max_mtiles(n_rows, E) + E + 2 * PF_XCD) * sizeof(int32_t), 256);
}

size_t prefill_ws_bytes(int n_rows, int E, int d) {
    return prefill_plan_bytes(n_rows, E) + prefill_split_bytes(n_rows, E, d);
}

// The generic kernels take more dynamic LDS than the default limit.  The
// attribute is raised once per device (std::call_once per device index, so
// concurrent first calls from several threads are safe); a failure is kept
// and returned by every later call on that device.
constexpr int PG_MAX_DEVICES = 64;
template <bool GATED>
static hipError_t generic_lds_attr() {
    static std::once_flag once[PG_MAX_DEVICES];
    static hipError_t result[PG_MAX_DEVICES];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= PG_MAX_DEVICES) return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev] {
        result[dev] = hipFuncSetAttribute((const void*)ffn_prefill_generic_kernel<GATED>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)PG_LDS_BYTES);
    });
    return result[dev];
}

// Shapes the tiled kernel takes: K a multiple of its 64-wide stages, N a
// multiple of 8 (its output leaves in 16-byte row chunks).
static bool pf_tiled_ok(int N, int K) { return K % PF_BK == 0 && N % 8 == 0; }

template <bool GATED>
static hipError_t launch_prefill_gemm(int n_rows, int N, int K, int n_nt, int max_mt, int bm, int E,
                                      const bf16* A, const int32_t* rowmap, int topk,
                                      const int32_t* mt_count,
                                      const int32_t* mt_expert, const int32_t* mt_row0,
                                      const int32_t* offsets, const bf16* Wa, const bf16* Wb,
                                      bf16* out, float* part, int32_t* claim, hipStream_t s) {
    // Workgroups for the plan's row tiles: the groups hold at most n_rows rows
    // (offsets is a prefix sum ending at or below n_rows), so there are at
    // most n_rows / bm full tiles plus one partly filled tile per expert.
    // The grid follows that bound rather than max_mt (sized for 128-row
    // tiles), since every workgroup past the real tiles is still dispatched,
    // at the end of the launch, only to exit.
    const long mts = std::min((long)max_mt, (long)n_rows / bm + E + 1);
    const long tiles = mts * n_nt;
    if (pf_tiled_ok(N, K)) {
        const int cus = prefill_cpx();  // compute units per XCD (0: unknown)
        // the second GEMM may cut its last round into k ranges (K >= 4 stages)
        const int cpx = (!GATED && K / PF_BK >= 4) ? cus : 0;
        // with claim counters, one more round of workgroups per XCD that can
        // take over tiles of the others' tails
        const int xc = claim != nullptr ? cus : 0;
        const unsigned grid = (unsigned)(((tiles + PF_XCD - 1) / PF_XCD + xc) * PF_XCD);
        const unsigned sgrid = (unsigned)(PF_XCD * cpx);  // split units: at most cpx per XCD
        if (bm == 256)
            ffn_prefill_kernel<GATED, 256, 5, false><<<grid, PF_THREADS, 0, s>>>(
                n_rows, N, K, n_nt, A, rowmap, topk, mt_count, mt_expert, mt_row0, offsets, Wa, Wb, out, cpx, part,
                claim, xc);
        else
            ffn_prefill_kernel<GATED, 128, 3, false><<<grid, PF_THREADS, 0, s>>>(
                n_rows, N, K, n_nt, A, rowmap, topk, mt_count, mt_expert, mt_row0, offsets, Wa, Wb, out, cpx, part,
                claim, xc);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess || cpx == 0 || GATED) return err;
        if (bm == 256)
            ffn_prefill_kernel<false, 256, 5, true><<<sgrid, PF_THREADS, 0, s>>>(
                n_rows, N, K, n_nt, A, rowmap, topk, mt_count, mt_expert, mt_row0, offsets, Wa, Wb, out, cpx, part,
                nullptr, 0);
        else
            ffn_prefill_kernel<false, 128, 3, true><<<sgrid, PF_THREADS, 0, s>>>(
                n_rows, N, K, n_nt, A, rowmap, topk, mt_count, mt_expert, mt_row0, offsets, Wa, Wb, out, cpx, part,
                nullptr, 0);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        const dim3 rgrid((unsigned)(PF_XCD * (cpx / 2)), (unsigned)(bm / PF_RD_ROWS));
        if (bm == 256)
            ffn_split_reduce_kernel<256><<<rgrid, 256, 0, s>>>(n_rows, N, n_nt, cpx, mt_count, mt_expert, mt_row0,
                                                               offsets, part, out);
        else
            ffn_split_reduce_kernel<128><<<rgrid, 256, 0, s>>>(n_rows, N, n_nt, cpx, mt_count, mt_expert, mt_row0,
                                                               offsets, part, out);
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)((((long)max_mt * n_nt + PF_XCD - 1) / PF_XCD) * PF_XCD);
    hipError_t aerr = generic_lds_attr<GATED>();
    if (aerr != hipSuccess) return aerr;
    ffn_prefill_generic_kernel<GATED><<<grid, PG_THREADS, PG_LDS_BYTES, s>>>(
        n_rows, N, K, n_nt, A, rowmap, topk, mt_count, mt_expert, mt_row0, offsets, Wa, Wb, out);
    return hipGetLastError();
}

// Row-tile height: 256 when the expert groups hold at least 128 rows on
// average, else 128.  Padded token blocks of a partly filled tile cost no
// MFMAs, so 256-row tiles lose little on groups of 128-256 rows, and they read
// each weight tile once per 256 rows instead of once per 128 (measured on the
// DeepSeek-V3-shaped layer, 128 rows per expert on average: gate/up 3.42 ->
// 3.28 ms).  The generic variant always uses 256-row tiles.
static int prefill_bm(int n_rows, int E, int d, int F) {
    if (!pf_tiled_ok(F, d) || !pf_tiled_ok(d, F)) return 256;
    return n_rows >= 128 * E ? 256 : 128;
}

hipError_t launch_ffn_prefill(int n_rows, int E, int d, int F, const void* A, const int32_t* rowmap,
                              int topk, const int32_t* offsets, const void* w1, const void* w3,
                              const void* w2, void* act, void* h, void* ws, hipStream_t s) {
    const int max_mt = prefill_max_mtiles(n_rows, E);
    const int bm = prefill_bm(n_rows, E, d, F);
    int32_t* mt_count = reinterpret_cast<int32_t*>(ws);
    int32_t* mt_expert = mt_count + 1;
    int32_t* mt_row0 = mt_expert + max_mt;
    int32_t* small_count = mt_row0 + max_mt;
    int32_t* small_list = small_count + 1;
    int32_t* claim = small_list + E;  // gate/up counters, then the second GEMM's
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + prefill_plan_bytes(n_rows, E));
    // With many experts some groups are small: those stream their weights
    // through the decode kernel instead of padding a row tile.
    const int small = (E >= PF_SMALL_MIN_E) ? DC_SMALL_ROWS : 0;
    MOE_TIMED_LAUNCH(MOE_KERNEL_FFN_PLAN, s,
                     ffn_plan_kernel<<<1, 1024, 0, s>>>(E, max_mt, bm, small, offsets, mt_count, mt_expert,
                                                        mt_row0, small_count, small_list, claim));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // The timing hook brackets each GEMM step as a whole: the tiled launch,
    // the small-expert launch and (second GEMM) the k-split launches.
    timer_before(MOE_KERNEL_FFN_GATE_UP, s);
    err = launch_prefill_gemm<true>(n_rows, F, d, (F + 127) / 128, max_mt, bm, E, (const bf16*)A,
                                    rowmap, topk, mt_count, mt_expert, mt_row0, offsets, (const bf16*)w1,
                                    (const bf16*)w3, (bf16*)act, nullptr, claim, s);
    if (err != hipSuccess) return err;
    if (small) {
        err = launch_small_experts(true, E, n_rows, F, d, A, rowmap, topk, offsets, small_list, small_count, w1,
                                   w3, act, s);
        if (err != hipSuccess) return err;
    }
    timer_after(MOE_KERNEL_FFN_GATE_UP, s);
    timer_before(MOE_KERNEL_FFN_DOWN, s);
    err = launch_prefill_gemm<false>(n_rows, d, F, (d + PF_BN - 1) / PF_BN, max_mt, bm, E,
                                     (const bf16*)act, nullptr, 1, mt_count, mt_expert, mt_row0, offsets,
                                     (const bf16*)w2, nullptr, (bf16*)h, part, claim + PF_XCD, s);
    if (err != hipSuccess) return err;
    if (small) {
        err = launch_small_experts(false, E, n_rows, d, F, act, nullptr, 1, offsets, small_list, small_count, w2,
                                   nullptr, h, s);
        if (err != hipSuccess) return err;
    }
    timer_after(MOE_KERNEL_FFN_DOWN, s);
    return hipSuccess;
}

// A plain linear layer (one group of n_rows rows) on the second GEMM's
// kernels: the tile plan for E = 1, then the tiled GEMM (with its last-round
// split).  Up to 64 rows stream W through the decode kernel instead.
size_t linear_ws_bytes(int n_rows, int N, int K) {
    return n_rows <= LIN_SMALL_ROWS ? linear_small_ws_bytes(n_rows, N, K) : prefill_ws_bytes(n_rows, 1, N);
}

hipError_t launch_linear(int n_rows, int N, int K, const void* x, const int32_t* offs, const void* w, void* y,
                         void* ws, hipStream_t s) {
    if (n_rows <= LIN_SMALL_ROWS) return launch_linear_small(n_rows, N, K, x, offs, w, y, ws, s);
    const int max_mt = prefill_max_mtiles(n_rows, 1);
    const int bm = !pf_tiled_ok(N, K) ? 256 : (n_rows >= 512 ? 256 : 128);
    int32_t* mt_count = reinterpret_cast<int32_t*>(ws);
    int32_t* mt_expert = mt_count + 1;
    int32_t* mt_row0 = mt_expert + max_mt;
    int32_t* small_count = mt_row0 + max_mt;
    int32_t* small_list = small_count + 1;
    float* part = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + prefill_plan_bytes(n_rows, 1));
    ffn_plan_kernel<<<1, 1024, 0, s>>>(1, max_mt, bm, 0, offs, mt_count, mt_expert, mt_row0, small_count,
                                       small_list, nullptr);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_prefill_gemm<false>(n_rows, N, K, (N + PF_BN - 1) / PF_BN, max_mt, bm, 1, (const bf16*)x, nullptr,
                                      1, mt_count, mt_expert, mt_row0, offs, (const bf16*)w, nullptr, (bf16*)y,
                                      part, nullptr, s);
}

}  // namespace moe
