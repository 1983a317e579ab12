// Microbenchmarks of the two machine limits the MoE kernels are measured
// against on the same GPU, next to the datasheet peaks:
//   * the HBM read rate a plain streaming kernel reaches (the bound of the
//     weight-streaming layers), and
//   * the bf16 rate of back-to-back v_mfma_f32_32x32x16_bf16 on register
//     operands with random bits (the bound of the compute-bound layers; the
//     clock the power limit allows depends on the operands' switching, so the
//     operands are random and rotate between instructions).
// Built as its own library (libmoepeaks.so); nothing in libmoe.so uses it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/moe_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;

// Workgroup b reads the contiguous 32 KB pieces b, b + gridDim.x, ... of the
// buffer: per piece each thread issues kStreamUnroll 16-byte loads 4 KB apart
// (all in flight at once), so every wave load covers 1 KB of consecutive
// bytes and a workgroup's loads stay inside one piece.  The XOR of everything
// a thread read goes to sink (one word per thread), so no load can be dropped.
constexpr size_t kPieceVec = (size_t)kStreamThreads * kStreamUnroll;  // 16-byte vectors per piece
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ buf, size_t n_vec,
                                                                     uint32_t* __restrict__ sink) {
    const size_t n_piece = n_vec / kPieceVec;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (size_t p = blockIdx.x; p < n_piece; p += gridDim.x) {
        const u32x4* q = buf + p * kPieceVec + threadIdx.x;
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = q[u * kStreamThreads];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
    }
    // the tail past the last whole piece
    const size_t tid = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
    for (size_t i = n_piece * kPieceVec + tid; i < n_vec; i += (size_t)gridDim.x * kStreamThreads) acc ^= buf[i];
    sink[tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

constexpr int kMfmaThreads = 256;
constexpr int kMfmaAcc = 8;   // independent accumulators (hide the MFMA latency)
constexpr int kMfmaOps = 4;   // operand fragments each side rotates through

// Every wave loads kMfmaOps random fragments per operand once, then runs
// iters rounds of kMfmaAcc independent 32x32x16 MFMAs whose operands rotate
// through them; one float per wave goes to sink.
__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(const u32x4* __restrict__ data, int iters,
                                                                 float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = (int)(blockIdx.x * (kMfmaThreads / 64) + threadIdx.x / 64);
    bf16x8 a[kMfmaOps], b[kMfmaOps];
#pragma unroll
    for (int j = 0; j < kMfmaOps; ++j) {
        a[j] = __builtin_bit_cast(bf16x8, data[((size_t)(wave % 64) * 2 * kMfmaOps + j) * 64 + lane]);
        b[j] = __builtin_bit_cast(bf16x8, data[((size_t)(wave % 64) * 2 * kMfmaOps + kMfmaOps + j) * 64 + lane]);
    }
    f32x16 acc[kMfmaAcc];
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.0f;
    // iters is a multiple of kMfmaOps, so the rotation is fixed at compile time
    for (int it = 0; it < iters; it += kMfmaOps) {
#pragma unroll
        for (int r = 0; r < kMfmaOps; ++r)
#pragma unroll
            for (int j = 0; j < kMfmaAcc; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + r) % kMfmaOps], b[(j / 2 + r) % kMfmaOps],
                                                                 acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[j][i];
    if (lane == 0) sink[wave] = s;
}

}  // namespace

extern "C" {

int peak_stream_read(const void* buf, size_t bytes, int blocks, uint32_t* sink, void* stream) {
    if (!buf || !sink || blocks <= 0 || bytes < 16 || ((uintptr_t)buf & 15u)) return 1;
    stream_read_kernel<<<blocks, kStreamThreads, 0, (hipStream_t)stream>>>((const u32x4*)buf, bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

size_t peak_stream_sink_words(int blocks) { return (size_t)blocks * kStreamThreads; }

int peak_mfma_loop(const void* data, int iters, int blocks, float* sink, void* stream) {
    if (!data || !sink || blocks <= 0 || iters <= 0 || iters % kMfmaOps || ((uintptr_t)data & 15u)) return 1;
    mfma_loop_kernel<<<blocks, kMfmaThreads, 0, (hipStream_t)stream>>>((const u32x4*)data, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

size_t peak_mfma_data_bytes(void) { return (size_t)64 * 2 * kMfmaOps * 64 * 16; }
size_t peak_mfma_sink_words(int blocks) { return (size_t)blocks * (kMfmaThreads / 64); }
double peak_mfma_flops(int iters, int blocks) {
    return (double)blocks * (kMfmaThreads / 64) * iters * kMfmaAcc * (2.0 * 32 * 32 * 16);
}

}  // extern "C"
