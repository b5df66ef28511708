// Skinny fp16 NT GEMM: C = A . B^T for 1 <= M <= 16 rows of A (the batch
// of a decode step: a few vectors against one large matrix B), fp32
// accumulation, fp16 out.
//
// Structure (TileLang GEMV page: GEMV as the degenerate GEMM whose A has a
// single row, K split over parallel workers and reduced at the end; here
// with up to 16 rows of A):
//  * B (N x K) dominates the traffic, so every byte of B is read once and
//    streamed: each MFMA v_mfma_f32_16x16x32_f16 takes 16 rows of B and the
//    (zero-padded) 16 rows of A over 32 k, both straight from global memory
//    into registers in the MFMA operand layout (lane l: row l % 16, k group
//    l / 16).  Nothing is shared between the waves of a workgroup except the
//    final reduction, so there is no LDS staging.
//  * A workgroup of W waves owns NB blocks of 16 rows of B; its waves split
//    K into W contiguous ranges (long runs along each row of B), each wave
//    keeping two batches of U k-steps of loads in flight.
//  * The W partial 16 x 16 tiles per block are summed in LDS in wave order
//    (deterministic) and rounded once to fp16.
// Requires K % 8 == 0 and 16-byte aligned A and B (the 16-byte loads).
#pragma once
#include "common.hpp"

namespace gf {

constexpr int kSkinnyMaxM = 16;

// One batch of U k-steps: the A and B fragments of steps s .. s+U-1 (zeros
// past the wave's range or past K; the address stays valid either way).
template <int NB, int U>
struct SkinnyBatch {
    half8 a[U], b[U][NB];

    __device__ __forceinline__ void load(const half8* ap, const half8* const (&bp)[NB], bool a_row,
                                         int s, int s_end, int kq, int K)
    {
        const half8 zero = {};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int ss = s + u;
            const bool ok = ss < s_end && ss * 32 + kq * 8 < K;
            const int off = ok ? ss * 4 : 0;     // in 8-element units
            a[u] = (ok && a_row) ? ap[off] : zero;
#pragma unroll
            for (int j = 0; j < NB; ++j) b[u][j] = ok ? __builtin_nontemporal_load(bp[j] + off) : zero;
        }
    }

    __device__ __forceinline__ void mma(floatx4 (&acc)[NB]) const
    {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[u], b[u][j], acc[j], 0, 0, 0);
    }
};

// NB 16-row blocks of B per workgroup, W waves splitting K, batches of U
// k-steps double-buffered in registers (the loads of batch i + 1 are in
// flight while batch i is multiplied).
template <int NB, int U, int W>
__global__ __launch_bounds__(W * kWave) void skinny_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C, int M,
    int N, int K)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __shared__ floatx4 part[W][NB][kWave];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int r = lane % 16, kq = lane / 16;   // operand row, 8-element K group
    const int n0 = blockIdx.x * NB * 16;
    const int steps = ceil_div(K, 32);
    const int per = ceil_div(steps, W);
    const int s_begin = min(steps, wave * per);
    const int s_end = min(steps, s_begin + per);
    const bool a_row = r < M;
    // Rows past M feed zeros; rows past N are clamped (loaded, never stored).
    const half8* ap = (const half8*)(A + (size_t)(a_row ? r : 0) * K + kq * 8);
    const half8* bp[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
        bp[j] = (const half8*)(B + (size_t)min(n0 + j * 16 + r, N - 1) * K + kq * 8);
    floatx4 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    SkinnyBatch<NB, U> b0, b1;
    b0.load(ap, bp, a_row, s_begin, s_end, kq, K);
    for (int s = s_begin; s < s_end; s += 2 * U) {
        b1.load(ap, bp, a_row, s + U, s_end, kq, K);
        b0.mma(acc);
        b0.load(ap, bp, a_row, s + 2 * U, s_end, kq, K);
        b1.mma(acc);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) part[wave][j][lane] = acc[j];
    __syncthreads();
    if (threadIdx.x < NB * kWave) {
        const int j = threadIdx.x / kWave, l = threadIdx.x % kWave;
        floatx4 sum = part[0][j][l];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += part[w][j][l];
        // Accumulator i of lane l holds row 4 * (l / 16) + i, column l % 16.
        const int n = n0 + j * 16 + l % 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (l / 16) + i;
            if (m < M && n < N) C[(size_t)m * N + n] = f32_to_f16_bits(sum[i]);
        }
    }
#endif
}

template <int NB, int U, int W>
hipError_t launch_skinny(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                         hipStream_t stream)
{
    const int grid = ceil_div(N, NB * 16);
    hipLaunchKernelGGL((skinny_kernel<NB, U, W>), dim3(grid), dim3(W * kWave), 0, stream, A, B, C,
                       M, N, K);
    return hipGetLastError();
}

}  // namespace gf
