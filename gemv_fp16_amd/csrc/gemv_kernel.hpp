// fp16 GEMV for gfx950: y = W . x with fp32 accumulation, no MFMA.
//
// The TileLang GEMV page walks a bandwidth-bound kernel from one thread per
// output to: K split across the threads of an output (reduce_threads), 128-bit
// vector loads (8 fp16 per load), and a tree reduction over the K-splitting
// threads in place of shared-memory atomics, with BLOCK_N x reduce_threads
// tuned.  The CDNA4 form here:
//  * one wave64 owns ROWS consecutive rows; its 64 lanes split K, lane l
//    taking the 16-byte chunks l, l+64, l+128, ... of every row;
//  * W is streamed with 128-bit non-temporal loads, UNROLL chunks per row
//    and lane in flight (ROWS * UNROLL loads per lane per step), x chunks are
//    loaded once per step and reused for all ROWS rows;
//  * fp16 pairs are multiplied and accumulated in fp32 with v_dot2_f32_f16;
//  * each row's 64 lane partials are folded inside the wave with DPP
//    (quad_perm, row_half_mirror, row_mirror) and four readlanes, so no LDS
//    and no barrier is needed; WAVES waves per workgroup only set how many
//    rows a workgroup covers.
#pragma once
#include "common.hpp"

namespace gf {


template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                 CTRL, 0xF, 0xF, false));
}

// Sum of v over the 64 lanes of the wave (the same value in every lane).
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]: pairs
    v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]: quads
    v += dpp_f32<0x141>(v);   // row_half_mirror: 8 lanes
    v += dpp_f32<0x140>(v);   // row_mirror: 16 lanes (one DPP row)
    const int b = __builtin_bit_cast(int, v);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}

// 8 fp16 products accumulated in fp32 through 4 v_dot2_f32_f16.  The chunks
// are kept as half8 and split with shufflevector: bit-casting single lanes of
// a 32-bit vector to half2 was seen to collapse all four operands to the
// first dword with this compiler.
__device__ __forceinline__ float dot8(half8 w, half8 x, float acc)
{
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(w, w, 0, 1), __builtin_shufflevector(x, x, 0, 1), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(w, w, 2, 3), __builtin_shufflevector(x, x, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(w, w, 4, 5), __builtin_shufflevector(x, x, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(w, w, 6, 7), __builtin_shufflevector(x, x, 6, 7), acc, false);
    return acc;
}

// ALIGNED: W and x 16-byte aligned and K % 8 == 0 (128-bit loads);
// otherwise element loads with bounds checks.
template <int ROWS, int UNROLL, int WAVES, bool ALIGNED>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ y, int N, int K)
{
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int row0 = (blockIdx.x * WAVES + wave) * ROWS;
    if (row0 >= N) return;   // whole wave leaves; the kernel has no barrier

    float acc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[r] = 0.0f;

    if constexpr (ALIGNED) {
        const int nch = K / 8;                                   // 16-byte chunks per row
        const half8* xv4 = (const half8*)x;
        const half8* wr[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r)
            wr[r] = (const half8*)(W + (size_t)min(row0 + r, N - 1) * K);

        int j = lane;
        constexpr int STEP = kWave * UNROLL;
        const int nfull = (nch / STEP) * STEP;
        for (; j < nfull; j += STEP) {
            half8 wv[ROWS][UNROLL], xv[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
                    wv[r][u] = __builtin_nontemporal_load(wr[r] + j + u * kWave);
                xv[u] = xv4[j + u * kWave];
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int r = 0; r < ROWS; ++r) acc[r] = dot8(wv[r][u], xv[u], acc[r]);
        }
        for (; j < nch; j += kWave) {                            // ragged end of the row
            const half8 xc = xv4[j];
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
                acc[r] = dot8(__builtin_nontemporal_load(wr[r] + j), xc, acc[r]);
        }
    } else {
        for (int k = lane; k < K; k += kWave) {
            const float xk = f16_bits_to_f32(x[k]);
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const int row = min(row0 + r, N - 1);
                acc[r] = fmaf(f16_bits_to_f32(W[(size_t)row * K + k]), xk, acc[r]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const float s = wave_sum(acc[r]);
        if (lane == r && row0 + r < N) y[row0 + r] = f32_to_f16_bits(s);
    }
}

template <int ROWS, int UNROLL, int WAVES, bool ALIGNED>
hipError_t launch_gemv(const uint16_t* W, const uint16_t* x, uint16_t* y, int N, int K,
                       hipStream_t stream)
{
    const int rows_per_block = ROWS * WAVES;
    const int blocks = ceil_div(N, rows_per_block);
    hipLaunchKernelGGL((gemv_kernel<ROWS, UNROLL, WAVES, ALIGNED>), dim3(blocks), dim3(WAVES * 64),
                       0, stream, W, x, y, N, K);
    return hipGetLastError();
}

}  // namespace gf
