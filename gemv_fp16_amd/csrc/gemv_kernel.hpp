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
//    (quad_perm, row_half_mirror, row_mirror) and four readlanes, so the
//    reduction needs no LDS and no barrier;
//  * with a bounded grid ("blocks"), a workgroup owns ROWS rows at a time and
//    its waves split K (all workgroups read one contiguous band of W), row
//    groups walked grid-stride, x staged in LDS once; shapes that do not
//    split evenly fall back to waves walking row groups grid-stride.
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
// otherwise element loads with bounds checks.  XLDS (aligned only): the
// workgroup first copies x into LDS (K * 2 bytes of dynamic LDS) and every
// row reads its x chunks from there instead of from L2.
// Row groups of ROWS rows are walked grid-stride, wave by wave: with a
// bounded grid the whole chip streams one contiguous band of W at a time and
// keeps a bounded amount of loads in flight, which is what HBM serves best.
template <int ROWS, int UNROLL, int WAVES, bool ALIGNED, bool XLDS>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ x,
                                                          uint16_t* __restrict__ y, int N, int K)
{
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    extern __shared__ __attribute__((aligned(16))) char gemv_smem[];

    const half8* xv4 = (const half8*)x;
    GF_LDS half8* xs = (GF_LDS half8*)gemv_smem;
    if constexpr (XLDS) {
        // Stage x once per workgroup; the only barrier in the kernel.
        const int nch = K / 8;
        for (int j = threadIdx.x; j < nch; j += WAVES * kWave) xs[j] = xv4[j];
        __syncthreads();
    }
    // x chunk j: from LDS (an LDS-space pointer, so that the read is a
    // ds_read and its wait does not also wait for the W loads in flight)
    // or from global memory.
    auto xchunk = [&](int j) __attribute__((always_inline)) {
        if constexpr (XLDS) return xs[j];
        else return xv4[j];
    };

    const int groups = (N + ROWS - 1) / ROWS;
    for (int gidx = blockIdx.x * WAVES + wave; gidx < groups; gidx += gridDim.x * WAVES) {
        const int row0 = gidx * ROWS;
        float acc[ROWS];
#pragma unroll
        for (int r = 0; r < ROWS; ++r) acc[r] = 0.0f;

        if constexpr (ALIGNED) {
            const int nch = K / 8;                                   // 16-byte chunks per row
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
                for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                    for (int r = 0; r < ROWS; ++r)
                        wv[r][u] = __builtin_nontemporal_load(wr[r] + j + u * kWave);
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) xv[u] = xchunk(j + u * kWave);
#pragma unroll
                for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                    for (int r = 0; r < ROWS; ++r) acc[r] = dot8(wv[r][u], xv[u], acc[r]);
            }
            for (; j < nch; j += kWave) {                            // ragged end of the row
                const half8 xc = xchunk(j);
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
}

constexpr int kGemvXldsMaxK = 32768;   // x staged in LDS up to 64 KiB

// 16-byte W loads per lane per task of the split kernel.
template <int ROWS, int UNROLL>
constexpr int ntasks_loads()
{
    return ROWS * UNROLL;
}

// Bounded-grid GEMV with the workgroup's waves splitting K.  A workgroup owns
// ROWS consecutive rows at a time (row groups walked grid-stride); wave w
// streams chunks [w * CPW, (w + 1) * CPW) of each row, CPW = K / 8 / WAVES,
// UNROLL * 64 chunks per step.  All workgroups together therefore read one
// contiguous band of W at a time (the order HBM serves best), instead of
// one stripe of every row in flight.  The loads of the next (row group,
// step) task are issued before the current one is multiplied, and in the
// steady-state loop they are issued unconditionally, so that the wait before
// each multiply leaves that next task's loads in flight (a load under a
// branch, or a read of x through a generic pointer, would make the compiler
// wait for every load first).  Per row group, each wave folds its partial
// sums with DPP and parks them in LDS; after the group's single barrier,
// wave 0 adds the WAVES partials in wave order (deterministic) and writes y.
// The LDS slots alternate between groups, so the next group's partials
// never overwrite slots wave 0 is still reading.  x is staged in LDS once,
// by direct-to-LDS loads issued before the first W loads.  Requires 16-byte
// alignment, K % 8 == 0, K <= kGemvXldsMaxK and
// (K / 8) % (WAVES * 64 * UNROLL) == 0.
template <int ROWS, int UNROLL, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemv_split_kernel(const uint16_t* __restrict__ W,
                                                                const uint16_t* __restrict__ x,
                                                                uint16_t* __restrict__ y, int N,
                                                                int K)
{
    constexpr int STEP = kWave * UNROLL;               // chunks of a row per wave per task
    constexpr int NT = WAVES * kWave;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    extern __shared__ __attribute__((aligned(16))) char gemv_smem[];
    GF_LDS float* red = (GF_LDS float*)gemv_smem;      // [2][WAVES][ROWS] partial sums
    GF_LDS half8* xs = (GF_LDS half8*)(gemv_smem + ((2 * WAVES * ROWS * 4 + 15) & ~15));

    const int nch = K / 8;
    const int cpw = nch / WAVES;                       // chunks per wave per row
    const int spg = cpw / STEP;                        // tasks per row group
    const int groups = (N + ROWS - 1) / ROWS;
    const int ngroups = (int)blockIdx.x < groups ? (groups - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
    const int ntasks = ngroups * spg;
    const int cbase = wave * cpw + lane;
    if (ntasks == 0) return;                           // no rows for this workgroup

    // x -> LDS: each wave instruction fills 64 consecutive 16-byte slots.
    for (int j0 = wave * kWave; j0 < nch; j0 += NT)
        if (j0 + lane < nch)
            __builtin_amdgcn_global_load_lds((const void*)((const half8*)x + j0 + lane),
                                             (GF_LDS void*)(xs + j0), 16, 0, 0);

    auto load = [&](int i, half8 (&b)[ROWS][UNROLL]) __attribute__((always_inline)) {
        const int g = blockIdx.x + (i / spg) * gridDim.x;
        const int s = i % spg;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const half8* wr = (const half8*)(W + (size_t)min(g * ROWS + r, N - 1) * K) + cbase + s * STEP;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) b[r][u] = __builtin_nontemporal_load(wr + u * kWave);
        }
    };
    half8 buf0[ROWS][UNROLL], buf1[ROWS][UNROLL];
    load(0, buf0);
    wait_vmcnt<ntasks_loads<ROWS, UNROLL>()>();        // x has landed; task 0's loads may fly
    lds_barrier();

    float acc[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) acc[r] = 0.0f;
    auto compute = [&](int i, const half8 (&b)[ROWS][UNROLL]) __attribute__((always_inline)) {
        const int s = i % spg;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const half8 xv = xs[cbase + s * STEP + u * kWave];
#pragma unroll
            for (int r = 0; r < ROWS; ++r) acc[r] = dot8(b[r][u], xv, acc[r]);
        }
        if (s == spg - 1) {                            // row group done
            const int gi = i / spg;
            GF_LDS float* slot = red + (gi & 1) * WAVES * ROWS;
#pragma unroll
            for (int r = 0; r < ROWS; ++r) {
                const float sum = wave_sum(acc[r]);
                if (lane == 0) slot[wave * ROWS + r] = sum;
                acc[r] = 0.0f;
            }
            lds_barrier();
            if (wave == 0 && lane < ROWS) {
                const int row = (blockIdx.x + gi * gridDim.x) * ROWS + lane;
                float t = 0.0f;
#pragma unroll
                for (int w = 0; w < WAVES; ++w) t += slot[w * ROWS + lane];
                if (row < N) y[row] = f32_to_f16_bits(t);
            }
        }
    };
    int i = 0;
    for (; i + 2 < ntasks; i += 2) {                   // tasks i + 1 and i + 2 exist
        load(i + 1, buf1);
        compute(i, buf0);
        load(i + 2, buf0);
        compute(i + 1, buf1);
    }
    if (i + 1 < ntasks) {
        load(i + 1, buf1);
        compute(i, buf0);
        compute(i + 1, buf1);
    } else if (i < ntasks) {
        compute(i, buf0);
    }
}

// blocks <= 0: one row group per wave (grid covers N); else at most `blocks`
// workgroups walking the row groups grid-stride.
template <int ROWS, int UNROLL, int WAVES, bool ALIGNED>
hipError_t launch_gemv(const uint16_t* W, const uint16_t* x, uint16_t* y, int N, int K, int blocks,
                       hipStream_t stream)
{
    const int rows_per_block = ROWS * WAVES;
    int grid = ceil_div(N, rows_per_block);
    if (blocks > 0 && grid > blocks) grid = blocks;
    if (ALIGNED && blocks > 0 && K > 0 && K <= kGemvXldsMaxK &&
        (K / 8) % (WAVES * 64 * UNROLL) == 0) {
        // Workgroup per row group, waves splitting K.
        int g2 = ceil_div(N, ROWS);
        if (g2 > blocks) g2 = blocks;
        const size_t lds = (size_t)2 * WAVES * ROWS * 4 + 32 + (size_t)K * 2;
        hipLaunchKernelGGL((gemv_split_kernel<ROWS, UNROLL, WAVES>), dim3(g2), dim3(WAVES * 64), lds,
                           stream, W, x, y, N, K);
    } else if (ALIGNED && blocks > 0 && K <= kGemvXldsMaxK) {
        // Each workgroup walks many row groups: stage x in LDS once.
        const size_t lds = (size_t)K * 2;
        hipLaunchKernelGGL((gemv_kernel<ROWS, UNROLL, WAVES, ALIGNED, ALIGNED>), dim3(grid),
                           dim3(WAVES * 64), lds, stream, W, x, y, N, K);
    } else {
        hipLaunchKernelGGL((gemv_kernel<ROWS, UNROLL, WAVES, ALIGNED, false>), dim3(grid),
                           dim3(WAVES * 64), 0, stream, W, x, y, N, K);
    }
    return hipGetLastError();
}

}  // namespace gf
