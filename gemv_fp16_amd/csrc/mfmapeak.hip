// MFMA throughput ceiling probe: a diagnostic program, not part of the
// library.  One wave per SIMD (256-thread workgroups, one per CU through
// 64 KiB of LDS) issues back-to-back independent v_mfma_f32_32x32x16_f16
// (16 accumulators x 4 per step, the GEMM kernel's 128 x 128 wave tile)
// for about 3 s; with the argument "sparse", the 2:4 sparse
// v_smfmac_f32_32x32x32_f16 instead (every lane's index fields name the
// pairs (0,1) (0,3) (1,2) (2,3), so all index values are valid), counted as
// 2 x 32 x 32 x 32 effective flops each.  Operands are fp16 values uniform in [-1, 1] (the GEMM
// workload's distribution: the matrix cores' power, and with it the clock
// the power limit allows, depends on the operand bits), read once from
// memory.  Reports TFLOP/s over wall time and the fraction of the
// shader-clock cycles the MFMA pipe was issuing, from s_memtime.
// Usage: ./mfmapeak
#include <hip/hip_runtime.h>
#include <cstdint>
#include <cstdio>
#include <utility>

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));

template <int I, int N, class F>
__device__ __forceinline__ void unroll_i(F&& f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        unroll_i<I + 1, N>(f);
    }
}

template <bool SPARSE>
__global__ __launch_bounds__(256) void mfma_stream(const half8* __restrict__ ops, float* out,
                                                   long long* cycles, int iters)
{
    extern __shared__ char lds_hold[];   // only reserves the CU
    (void)lds_hold;
    const int lane = threadIdx.x % 64;
    half8 a[4], b[4], b2[4];
    unroll_i<0, 4>([&](auto i) {
        a[decltype(i)::value] = ops[(decltype(i)::value * 64 + lane) % 512];
        b[decltype(i)::value] = ops[(256 + decltype(i)::value * 64 + lane) % 512];
        b2[decltype(i)::value] = ops[(384 + decltype(i)::value * 64 + lane) % 512];
    });
    const int idx = 0xE9C4;
    floatx16 acc[16];
    unroll_i<0, 16>([&](auto i) { acc[decltype(i)::value] = floatx16{}; });
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
        unroll_i<0, 4>([&](auto) {
            unroll_i<0, 16>([&](auto i) {
                constexpr int j = decltype(i)::value;
                if constexpr (SPARSE) {
                    const half16 bb = __builtin_shufflevector(b[j % 4], b2[j % 4], 0, 1, 2, 3, 4, 5, 6, 7, 8,
                                                              9, 10, 11, 12, 13, 14, 15);
                    acc[j] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(a[j / 4], bb, acc[j], idx, 0, 0);
                } else {
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j / 4], b[j % 4], acc[j], 0, 0, 0);
                }
            });
        });
    }
    const long long t1 = clock64();
    float s = 0.0f;
    unroll_i<0, 16>([&](auto i) { s += acc[decltype(i)::value][0]; });
    out[blockIdx.x * 256 + threadIdx.x] = s;
    if (lane == 0) cycles[blockIdx.x * 4 + threadIdx.x / 64] = t1 - t0;
}

int main(int argc, char** argv)
{
    const bool sparse = argc > 1 && argv[1][0] == 's';
    auto kern = sparse ? mfma_stream<true> : mfma_stream<false>;
    const int grid = 256, iters = 20000, reps = 150;   // 64 MFMA x 32 cycles per iteration
    // 512 fp16 operands uniform in [-1, 1]: a 64-bit LCG (Knuth's MMIX
    // constants), top 24 bits -> [0, 1), then 2u - 1 rounded to fp16.
    half8 host[512];
    uint64_t x = 1;
    for (int i = 0; i < 512; ++i)
        for (int e = 0; e < 8; ++e) {
            x = x * 6364136223846793005ull + 1442695040888963407ull;
            host[i][e] = (_Float16)(2.0f * (float)(x >> 40) / 16777216.0f - 1.0f);
        }
    half8* ops;
    float* out;
    long long* cyc;
    if (hipMalloc(&ops, sizeof(host)) != hipSuccess || hipMalloc(&out, grid * 256 * sizeof(float)) != hipSuccess ||
        hipMalloc(&cyc, grid * 4 * sizeof(long long)) != hipSuccess)
        return 1;
    if (hipMemcpy(ops, host, sizeof(host), hipMemcpyHostToDevice) != hipSuccess) return 1;
    if (hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 65536) !=
        hipSuccess)
        return 1;
    hipEvent_t e0, e1;
    (void)hipEventCreate(&e0);
    (void)hipEventCreate(&e1);
    for (int w = 0; w < 20; ++w)
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 65536, 0, ops, out, cyc, iters);
    (void)hipEventRecord(e0);
    for (int r = 0; r < reps; ++r)
        hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 65536, 0, ops, out, cyc, iters);
    (void)hipEventRecord(e1);
    if (hipEventSynchronize(e1) != hipSuccess) return 1;
    float ms = 0.0f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    static long long h[grid * 4];
    if (hipMemcpy(h, cyc, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return 1;
    double avg = 0.0;
    for (int i = 0; i < grid * 4; ++i) avg += (double)h[i];
    avg /= grid * 4;
    const double flop = 2.0 * 32 * 32 * (sparse ? 32 : 16) * 64 * (double)iters * grid * 4 * reps;
    const double sec = ms * 1e-3;
    printf("%s, uniform[-1,1] operands, one wave per SIMD: %.1f TFLOP/s over %.2f s "
           "(%.1f %% of %s), MFMA issue %.1f %% of shader cycles, mean shader clock %.2f GHz\n",
           sparse ? "smfmac 32x32x32 f16 (2:4, effective flops)" : "mfma 32x32x16 f16", flop / sec / 1e12, sec,
           flop / sec / 1e12 / (sparse ? 50.0 : 25.0), sparse ? "5000" : "2500", 2048.0 * iters / avg * 100.0,
           avg * reps / sec / 1e9);
    return hipDeviceSynchronize() != hipSuccess;
}
