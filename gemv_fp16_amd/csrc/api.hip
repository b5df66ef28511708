// C-ABI entry points: argument validation, config choice and launches.
// Validation runs entirely on the host before any HIP call, so invalid
// arguments never touch the device.
#include <stdint.h>
#include <string.h>

#include "../../include/gemvfp16.h"
#include "configs.hpp"
#include "gemv_kernel.hpp"
#include "skinny_kernel.hpp"

namespace gf {

GemmLaunchFn g_gemm_table[kNumGemm][6] = {};
GemmLaunchFn g_gemm_layout_table[kNumGemm][4][2] = {};

namespace {

constexpr int kDefaultPanel = 10;   // tile-rows per raster panel when raster == 1
constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int validate_gemm(const void* A, const void* B, const void* C, int M, int N, int K, int c_align)
{
    if (M < 0 || N < 0 || K < 0) return GF_ERR_INVALID_ARG;
    if ((int64_t)M * K > kMaxElems || (int64_t)N * K > kMaxElems || (int64_t)M * N > kMaxElems)
        return GF_ERR_INVALID_ARG;
    if (M > 0 && K > 0 && (!A || !aligned(A, 2))) return GF_ERR_INVALID_ARG;
    if (N > 0 && K > 0 && (!B || !aligned(B, 2))) return GF_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && (!C || !aligned(C, c_align))) return GF_ERR_INVALID_ARG;
    return GF_OK;
}

int find_gemm(const gf_gemm_cfg& c)
{
    for (int i = 0; i < kNumGemm; ++i) {
        const GemmDesc& d = kGemmConfigs[i];
        if (d.bm == c.block_m && d.bn == c.block_n && d.bk == c.block_k && d.stages == c.stages &&
            d.threads == c.threads && d.sched == c.schedule)
            return i;
    }
    return -1;
}

int panel_of(int raster) { return raster <= 0 ? 0 : (raster == 1 ? kDefaultPanel : raster); }

gf_gemm_cfg make_cfg(int bm, int bn, int bk, int s, int t, int raster, int sched = 0)
{
    gf_gemm_cfg c;
    c.block_m = bm; c.block_n = bn; c.block_k = bk; c.stages = s; c.threads = t; c.raster = raster;
    c.schedule = sched;
    return c;
}

// The tile config for a shape: the largest tile that still gives every CU a
// workgroup, in the form measured fastest for it (offline tile sweeps, then
// candidates timed side by side, alternating batch by batch).
//  * At least 256 tiles of 256 x 256:
//    - K > 1536: 256 x 256 x 64, two stages, one wave per SIMD (schedule 2),
//      first in the sweeps at M = N = 8192 for K = 4096 and 8192 and up to
//      4 % ahead of the 8-wave kernel side by side; grouped, XCD-aware tile
//      order (panels of 10 tile-rows) up to K = 4096 (5 % ahead at K = 1024,
//      tied at 4096), plain order up to K = 12288 (at 8192 panels of 2-10
//      rows are 0.2-1.8 % behind it, at 12288 all within noise), and from
//      K = 16384 the XCD-aware order with panels of 4 tile-rows, which makes
//      each XCD's share one panel (1.7-2.0 % ahead of the plain order at
//      16384 in three side-by-side runs; 0.3 % at 32768).
//    - K <= 1536 (timed at K = 128 .. 4096 on 8192^2, and at 4096^2, 6144^2,
//      8192 x 4096 and 16384 x 8192): 512-thread tiles.  Up to K = 512 the
//      C write outweighs the operand reads (8x at K = 256), and tiles that
//      leave room for more than one workgroup per CU overlap one
//      workgroup's epilogue with another's main loop: 128 x 256 x 32 with
//      three stages at K <= 256 given at least 1024 of them (1.24-1.61x),
//      else 256 x 128 x 64 with one stage (1.12-1.27x).  Up to K = 1536, the
//      8-wave 256 x 256 kernel in plain order (1.03-1.10x; even at 2048).
//  * Fewer (tile sweeps at 2048 x 4096, 2048 x 2048 and 1024 x 4096 x 8192;
//    candidates at ten mid-size shapes with K = 1024 .. 8192):
//    - 256 x 128 once 256 of them fill the CUs, given K >= 2048: below that
//      the per-workgroup start and epilogue weigh more, and two 128 x 128
//      workgroups per CU hide them;
//    - 128 x 128 with four stages (one workgroup per CU) while one round of
//      them covers the shape (for K <= 512, 64 x 128 with two stages
//      instead: 1.17-1.41x at six shapes), two stages (two per CU, one
//      round of 512) past it;
//    - below 128 of those, 64 x 64 with three stages: 1.5-1.9x the
//      two-stage form at every small shape measured (M = 32 .. 1024,
//      K = 1024 .. 8192).
// Every tile chosen here is compiled with its masked variant too, so
// unaligned operands run the same tile.
gf_gemm_cfg default_gemm_cfg(int M, int N, int K)
{
    const int64_t t256 = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
    const int64_t t25612 = (int64_t)ceil_div(M, 256) * ceil_div(N, 128);
    const int64_t t128 = (int64_t)ceil_div(M, 128) * ceil_div(N, 128);
    if (t256 >= 256) {
        const int64_t t12825 = (int64_t)ceil_div(M, 128) * ceil_div(N, 256);
        if (K <= 256 && t12825 >= 1024) return make_cfg(128, 256, 32, 3, 512, 0);
        if (K <= 512) return make_cfg(256, 128, 64, 1, 512, 0);
        if (K <= 1536) return make_cfg(256, 256, 64, 2, 512, 0);
        return make_cfg(256, 256, 64, 2, 256, K <= 4096 ? 1 : (K < 16384 ? 0 : 4), 2);
    }
    if (t25612 >= 256 && K >= 2048) return make_cfg(256, 128, 64, 3, 256, 0, 2);
    if (t128 >= 128 && t128 <= 256)
        return K <= 512 ? make_cfg(64, 128, 64, 2, 256, 0) : make_cfg(128, 128, 64, 4, 256, 0, 2);
    if (t128 > 256) return make_cfg(128, 128, 64, 2, 256, 0);
    return make_cfg(64, 64, 64, 3, 256, 0);
}

// Wave quantisation of the default tile.  One 256 x 256 workgroup fills a
// CU, so the tiles run in rounds of 256; when the last round is at most half
// full (7168^2: 784 tiles = 3 rounds + 16 tiles, and those 16 take as long as
// a full round), the leading tile-rows that fill whole rounds run as one
// launch and the remaining rows (at most 1024) as a second launch with a
// tile that spreads them over the chip.  Returns the row count of the first
// part; M means no split.  A and C rows are contiguous, so both parts are
// ordinary launches on row ranges, and every output of a 128 x 128 tail is
// computed by the same 32 x 32 MFMAs over K in the same order as with the
// big tile: the result does not depend on the split.
int row_split(int M, int N, const gf_gemm_cfg& big)
{
    constexpr int64_t kCus = 256, kMaxTailRows = 1024;
    if (big.block_m != 256 || big.block_n != 256) return M;
    const int64_t tn = ceil_div(N, 256), tiles = (int64_t)ceil_div(M, 256) * tn;
    const int64_t rounds = (tiles + kCus - 1) / kCus;
    if (rounds < 2 || tiles - kCus * (rounds - 1) > kCus / 2) return M;
    const int64_t m1 = (kCus * (rounds - 1) / tn) * 256;
    if (m1 < 256 || m1 >= M || M - m1 > kMaxTailRows) return M;
    return (int)m1;
}

// Tile of the rows past the split: 128 x 128 tiles, four stages when one
// round of them covers the rows, else two stages (two workgroups per CU).
gf_gemm_cfg tail_gemm_cfg(int M, int N)
{
    const int64_t t128 = (int64_t)ceil_div(M, 128) * ceil_div(N, 128);
    return t128 <= 256 ? make_cfg(128, 128, 64, 4, 256, 0, 2) : make_cfg(128, 128, 64, 2, 256, 0, 2);
}

// Split-K tile: the largest tile (among the configs compiled with the fp32
// epilogues) whose tiles x slices still give every CU a workgroup.  Sweeps
// of every such config at M = N = 1024, K = 16384 with the operands rotated
// through HBM found exactly that for the two-pass combines: 128 x 128 with
// 3 stages at split 4 (714-727 TFLOP/s), 256 x 128 with one wave per SIMD
// at split 8 (711-715, against 562-567 for the 128 x 256 tile it
// replaces), 256 x 256 at split 16 (609-635), each with 256 workgroups.
// The atomic combine gathers 16 partial tiles on every output tile at split
// 16 when those tiles are 256 x 256, and their adds arrive together; there
// the 64 x 64 tile spreads them over 16 rounds of workgroups (455 against
// 393 TFLOP/s).  So with atomics, wherever the big tiles would stack 16 or
// more slices, the 64 x 64 tile is taken.
gf_gemm_cfg default_splitk_cfg(int M, int N, int K, int split_k, bool atomic = false)
{
    constexpr int kCus = 256;
    const gf_gemm_cfg cands[] = {
        make_cfg(256, 256, 64, 2, 512, 1), make_cfg(256, 128, 64, 3, 256, 1, 2),
        make_cfg(128, 128, 64, 3, 256, 1), make_cfg(64, 64, 64, 3, 256, 1),
    };
    constexpr int kLast = sizeof(cands) / sizeof(cands[0]) - 1;
    for (int i = 0; i <= kLast; ++i) {
        const gf_gemm_cfg& c = cands[i];
        const int64_t tiles = (int64_t)ceil_div(M, c.block_m) * ceil_div(N, c.block_n);
        const int nkt = ceil_div(K, c.block_k);
        const int per = nkt > 0 ? ceil_div(nkt, max(1, split_k)) : 0;
        const int slices = per > 0 ? ceil_div(nkt, per) : 1;
        if (tiles * slices >= kCus) return atomic && slices >= 16 ? cands[kLast] : c;
    }
    return cands[kLast];
}

int launch_status(hipError_t e) { return e == hipSuccess ? GF_OK : GF_ERR_HIP; }

// Whether the 128-bit operand path applies: 16-byte aligned A and B, K % 8 == 0.
bool operands_aligned(const void* A, const void* B, int K)
{
    return aligned(A, 16) && aligned(B, 16) && (K % 8 == 0);
}

// One GEMM launch of epilogue `epi` over `slices` K slices of kt_per tiles.
int run_gemm(const void* A, const void* B, void* C, int M, int N, int K, const gf_gemm_cfg& cfg,
             int epi, int slices, int kt_per, bool c16_aligned, hipStream_t stream)
{
    const int idx = find_gemm(cfg);
    if (idx < 0) return GF_ERR_UNSUPPORTED;
    const bool al = operands_aligned(A, B, K) && c16_aligned;
    GemmLaunchFn fn = g_gemm_table[idx][epi * 2 + (al ? 1 : 0)];
    if (!fn) return GF_ERR_UNSUPPORTED;
    GemmArgs a;
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.C = C;
    a.M = M; a.N = N; a.K = K;
    a.kt_per_slice = kt_per;
    a.raster = panel_of(cfg.raster);
    return launch_status(fn(a, slices, stream));
}

__global__ void zero_f32_kernel(float* __restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = i; t < n; t += stride) p[t] = 0.0f;
}

__global__ void zero_f32x4_kernel(floatx4* __restrict__ p, int64_t n4)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = i; t < n4; t += stride) p[t] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
}

// Slices s0 .. s0+NB-1 of element t (slice s at ws[s * stride + t]) added
// to acc in ascending s; every load is issued before the first add, so a
// thread keeps NB requests in flight instead of waiting out each load's
// latency in turn.
template <int NB, class V>
__device__ __forceinline__ V add_slices(V acc, const V* __restrict__ ws, int64_t stride, int64_t t,
                                        int s0)
{
    V v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) v[j] = ws[(int64_t)(s0 + j) * stride + t];
#pragma unroll
    for (int j = 0; j < NB; ++j) acc += v[j];
    return acc;
}

// The slices of element t summed in fp32 in ascending s from +0: the fixed
// order that makes the two-pass result reproducible.  (A partial is an MFMA
// sum that started from +0, so it is never -0, and +0 + p == p: the sum
// equals the one that starts from slice 0 itself.)  Loads go out 8 slices
// at a time.
template <class V>
__device__ __forceinline__ V sum_slices(const V* __restrict__ ws, int64_t stride, int64_t t, int slices)
{
    V acc = {};
    int s0 = 0;
    for (; s0 + 8 <= slices; s0 += 8) acc = add_slices<8>(acc, ws, stride, t, s0);
    switch (slices - s0) {
    case 1: return add_slices<1>(acc, ws, stride, t, s0);
    case 2: return add_slices<2>(acc, ws, stride, t, s0);
    case 3: return add_slices<3>(acc, ws, stride, t, s0);
    case 4: return add_slices<4>(acc, ws, stride, t, s0);
    case 5: return add_slices<5>(acc, ws, stride, t, s0);
    case 6: return add_slices<6>(acc, ws, stride, t, s0);
    case 7: return add_slices<7>(acc, ws, stride, t, s0);
    default: return acc;
    }
}

// C32[i] = sum over s = 0 .. slices-1, ascending, of ws[s][i].
__global__ void splitk_reduce_x4_kernel(const floatx4* __restrict__ ws, floatx4* __restrict__ c,
                                        int64_t n4, int slices)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = i; t < n4; t += stride) c[t] = sum_slices(ws, n4, t, slices);
}

__global__ void splitk_reduce_kernel(const float* __restrict__ ws, float* __restrict__ c, int64_t n,
                                     int slices)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = i; t < n; t += stride) c[t] = sum_slices(ws, n, t, slices);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi)
{
    return f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
}

// C16[i] = fp16_rne(sum over s = 0 .. slices-1, ascending, of ws[s][i]):
// the fp32 sum of the two-pass reduce, rounded once.  Eight outputs (two
// float4 per slice in, one 16-byte store out) per thread.
__global__ void splitk_reduce_f16x8_kernel(const floatx4* __restrict__ ws, u32x4* __restrict__ c,
                                           int64_t n8, int slices)
{
    typedef float floatx8 __attribute__((ext_vector_type(8)));
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = i; t < n8; t += stride) {
        const floatx8 v = sum_slices((const floatx8*)ws, n8, t, slices);
        u32x4 o;
        o.x = pack_f16x2(v[0], v[1]);
        o.y = pack_f16x2(v[2], v[3]);
        o.z = pack_f16x2(v[4], v[5]);
        o.w = pack_f16x2(v[6], v[7]);
        c[t] = o;
    }
}

__global__ void splitk_reduce_f16_kernel(const float* __restrict__ ws, uint16_t* __restrict__ c,
                                         int64_t n, int slices)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = i; t < n; t += stride) c[t] = f32_to_f16_bits(sum_slices(ws, n, t, slices));
}

__global__ void zero_u16_kernel(uint16_t* __restrict__ p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = i; t < n; t += stride) p[t] = 0;
}

int grid_for(int64_t n, int block)
{
    int64_t g = (n + block - 1) / block;
    if (g > 8192) g = 8192;
    return (int)(g < 1 ? 1 : g);
}

int zero_f32(float* p, int64_t n, hipStream_t stream)
{
    if (aligned(p, 16) && n % 4 == 0) {
        hipLaunchKernelGGL(zero_f32x4_kernel, dim3(grid_for(n / 4, 256)), dim3(256), 0, stream,
                           reinterpret_cast<floatx4*>(p), n / 4);
    } else {
        hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(n, 256)), dim3(256), 0, stream, p, n);
    }
    return launch_status(hipGetLastError());
}

// Scratch for the entry point that allocates nothing: the two-pass slice
// partials of gemm_f16_nt_splitk_noalloc.  A file-scope device array, so the
// code object carries it and each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host that name is only a stand-in for the symbol): it takes
// the device address hipGetSymbolAddress returns, once per device, and uses
// that.  Every call on one GPU shares the array.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// The address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream), looked up with that device current on
// the first call there and kept.
int scratch_for_stream(hipStream_t stream, void** out)
{
    int cur = -1, dev = -1;
    if (hipGetDevice(&cur) != hipSuccess) return GF_ERR_HIP;
    dev = cur;
    if (stream) {
        hipDevice_t d;
        if (hipStreamGetDevice(stream, &d) != hipSuccess) return GF_ERR_HIP;
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxDevices) return GF_ERR_HIP;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return GF_ERR_HIP;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur && hipSetDevice(cur) != hipSuccess) return GF_ERR_HIP;
        if (e != hipSuccess || !p) return GF_ERR_HIP;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return GF_OK;
}

// The slice sums of a two-pass workspace into C32 (fp32) or C16 (fp16).
int splitk_reduce(const void* ws, void* C, bool out_f16, int64_t mn, int slices, hipStream_t stream)
{
    if (!out_f16 && aligned(ws, 16) && aligned(C, 16) && mn % 4 == 0) {
        hipLaunchKernelGGL(splitk_reduce_x4_kernel, dim3(grid_for(mn / 4, 256)), dim3(256), 0, stream,
                           static_cast<const floatx4*>(ws), static_cast<floatx4*>(C), mn / 4, slices);
    } else if (!out_f16) {
        hipLaunchKernelGGL(splitk_reduce_kernel, dim3(grid_for(mn, 256)), dim3(256), 0, stream,
                           static_cast<const float*>(ws), static_cast<float*>(C), mn, slices);
    } else if (aligned(ws, 32) && aligned(C, 16) && mn % 8 == 0) {   // 8-float vectors of ws
        hipLaunchKernelGGL(splitk_reduce_f16x8_kernel, dim3(grid_for(mn / 8, 256)), dim3(256), 0,
                           stream, static_cast<const floatx4*>(ws), static_cast<u32x4*>(C), mn / 8,
                           slices);
    } else {
        hipLaunchKernelGGL(splitk_reduce_f16_kernel, dim3(grid_for(mn, 256)), dim3(256), 0, stream,
                           static_cast<const float*>(ws), static_cast<uint16_t*>(C), mn, slices);
    }
    return launch_status(hipGetLastError());
}

// Tile-aligned split-K slices: kt_per K tiles each; only non-empty slices
// run (slices == 0 for K == 0).
void slice_plan(int K, int block_k, int split_k, int& kt_per, int& slices)
{
    const int nkt = ceil_div(K, block_k);
    kt_per = nkt > 0 ? ceil_div(nkt, split_k) : 0;
    slices = nkt > 0 ? ceil_div(nkt, kt_per) : 0;
}

int splitk_impl(const void* A, const void* B, float* C32, int M, int N, int K, int split_k,
                int mode, void* ws, size_t ws_bytes, const gf_gemm_cfg& cfg, hipStream_t stream)
{
    int rc = validate_gemm(A, B, C32, M, N, K, 4);
    if (rc) return rc;
    if (split_k < 1 || split_k > 65535) return GF_ERR_INVALID_ARG;
    if (mode != GF_SPLITK_ATOMIC && mode != GF_SPLITK_TWOPASS) return GF_ERR_INVALID_ARG;
    const int64_t mn = (int64_t)M * N;
    if (mode == GF_SPLITK_TWOPASS) {
        if ((uint64_t)ws_bytes < (uint64_t)split_k * (uint64_t)mn * sizeof(float)) return GF_ERR_INVALID_ARG;
        if (mn > 0 && (!ws || !aligned(ws, 4))) return GF_ERR_INVALID_ARG;
    }
    if (find_gemm(cfg) < 0) return GF_ERR_UNSUPPORTED;
    if (mn == 0) return GF_OK;

    int kt_per, slices;
    slice_plan(K, cfg.block_k, split_k, kt_per, slices);
    if (mode == GF_SPLITK_ATOMIC || slices == 0) {
        rc = zero_f32(C32, mn, stream);
        if (rc || slices == 0) return rc;
        return run_gemm(A, B, C32, M, N, K, cfg, EPI_F32_ATOMIC, slices, kt_per, true, stream);
    }
    rc = run_gemm(A, B, ws, M, N, K, cfg, EPI_F32_STORE, slices, kt_per, true, stream);
    if (rc) return rc;
    return splitk_reduce(ws, C32, false, mn, slices, stream);
}

// Split-K with an fp16 output: pass 1 stores each slice's fp32 partial tile
// into the workspace, pass 2 sums the slices in ascending order and rounds
// the sum once to fp16.
int splitk_f16_impl(const void* A, const void* B, void* C, int M, int N, int K, int split_k,
                    void* ws, size_t ws_bytes, const gf_gemm_cfg& cfg, hipStream_t stream)
{
    int rc = validate_gemm(A, B, C, M, N, K, 2);
    if (rc) return rc;
    if (split_k < 1 || split_k > 65535) return GF_ERR_INVALID_ARG;
    const int64_t mn = (int64_t)M * N;
    if ((uint64_t)ws_bytes < (uint64_t)split_k * (uint64_t)mn * sizeof(float)) return GF_ERR_INVALID_ARG;
    if (mn > 0 && (!ws || !aligned(ws, 4))) return GF_ERR_INVALID_ARG;
    if (find_gemm(cfg) < 0) return GF_ERR_UNSUPPORTED;
    if (mn == 0) return GF_OK;

    int kt_per, slices;
    slice_plan(K, cfg.block_k, split_k, kt_per, slices);
    if (slices == 0) {                           // K == 0: the empty sum
        hipLaunchKernelGGL(zero_u16_kernel, dim3(grid_for(mn, 256)), dim3(256), 0, stream,
                           static_cast<uint16_t*>(C), mn);
        return launch_status(hipGetLastError());
    }
    rc = run_gemm(A, B, ws, M, N, K, cfg, EPI_F32_STORE, slices, kt_per, true, stream);
    if (rc) return rc;
    return splitk_reduce(ws, C, true, mn, slices, stream);
}

int find_skinny(const gf_skinny_cfg& c)
{
    for (int i = 0; i < kNumSkinny; ++i)
        if (kSkinnyConfigs[i].blocks == c.blocks && kSkinnyConfigs[i].unroll == c.unroll &&
            kSkinnyConfigs[i].waves == c.waves && kSkinnyConfigs[i].stages == c.stages)
            return i;
    return -1;
}

// Skinny launch shape, from sweeps of the compiled shapes for M = 1..16 at
// N x K = 8192^2, 4096^2, 4096 x 14336, 2048 x 8192, 6144^2, 4096 x 11008,
// 8192 x 4096, 14336 x 4096, 16384 x 4096, 28672 x 4096, 8192 x 2048,
// 16384 x 2048 and 12288 x 6144, and side-by-side timings of the split form:
//  * split form (M <= 8, K = 8192 or 16384, at least 4096 rows of B): the
//    GEMV's split launch shape with A in registers (below);
//  * vector form (M <= 8): 8-wave workgroups where rows are long (K >= 8192)
//    or B is small; otherwise 16 waves with 4 chunks per lane in flight, for
//    M <= 2 over at least 32 M elements of B and for M <= 4 from 8192 rows
//    of B.  The 16-wave form also covers K not a multiple of 4096, where the
//    8-chunk form does not fit.
//  * LDS form (K % 512 == 0) from M = 5 below 8192 rows of B, with one
//    16-row block per workgroup (three blocks give 86 workgroups at
//    N = 4096); from 8192 rows for M > 8, or M > 4 at K <= 2048, with one
//    block per workgroup up to K = 4096 (two up to 2048) and three beyond.
gf_skinny_cfg default_skinny_cfg(int M, int N, int K)
{
    gf_skinny_cfg c;
    c.waves = 8;
    if (M > kSkinnyMaxM) {
        // 17 .. 64 rows: the LDS form with A in 16-row blocks (timed against
        // the tiles and each other at N x K = 8192^2, 4096 x 14336,
        // 2048 x 8192, 4096^2 and 1024 x 4096): three 16-row blocks of B
        // per workgroup at 8192 rows of B up to M = 32, two up to 48, else
        // one; below 8192 rows one block, three stages up to M = 32.
        c.unroll = 0;
        if (N >= 8192) {
            c.blocks = M <= 32 ? 3 : (M <= 48 ? 2 : 1);
            c.stages = 2;
        } else {
            c.blocks = 1;
            c.stages = M <= 32 ? 3 : 2;
        }
        return c;
    }
    // Split form (the GEMV's split launch shape, A in registers) where K is
    // 8192 or 16384 and B has at least 4096 rows, timed side by side against
    // the vector and LDS forms with B rotated through HBM at N x K = 8192^2,
    // 16384 x 8192, 4096 x 16384 and 8192 x 16384 (M = 1, 2, 4, 8):
    // 1.04-1.21x at K = 8192 (4 waves, 4 chunks per lane, 512 workgroups),
    // 1.07-1.30x at K = 16384 for M <= 4 (4 waves, 8 chunks) and 1.03-1.09x
    // there for M = 5..8 (8 waves, 4 chunks, 256 workgroups).  At K = 4096 it trails the vector
    // form (shorter rows: more reduction and barrier per byte).
    if (M <= kSkinnySplitMaxM && N >= 4096 && (K == 8192 || K == 16384)) {
        if (K == 8192) { c.blocks = 512; c.unroll = 4; c.waves = 4; }
        else if (M <= 4) { c.blocks = 512; c.unroll = 8; c.waves = 4; }
        else { c.blocks = 256; c.unroll = 4; c.waves = 8; }
        c.stages = -1;
        return c;
    }
    const bool small_n = N < 8192;
    const bool lds_ok = K > 0 && K % kSkinnyKc == 0;
    const bool lds_first = lds_ok && M > 4 && (small_n || K <= 2048);
    if (M <= kSkinnyVecMaxM && !lds_first) {
        const int unroll = M <= 2 ? 8 : 4;      // chunks in flight per lane in 8-wave workgroups
        const bool fits_8w = skinny_vec_fits(M, K, unroll) && skinny_vec_whole(K, unroll);
        const bool wants_16w = skinny_vec_fits(M, K, 4) && skinny_vec_whole(K, 4) &&
                               (M <= 2 ? (int64_t)N * K >= (int64_t)32 << 20 : M <= 4 && !small_n);
        if (fits_8w && (K >= 8192 || !wants_16w)) {
            c.blocks = 1;
            c.unroll = unroll;
            c.stages = 1;
            return c;
        }
        if (wants_16w) {
            c.blocks = 1;
            c.unroll = 4;
            c.waves = 16;
            c.stages = 1;
            return c;
        }
        // Rows that do not split into whole 2048-chunk steps (K = 11008,
        // 13824, 15360, 5120, ...): the vector form with a ragged last step
        // where at most a quarter of the last step's lanes are padding,
        // against the direct form it replaces 1.22-1.81x for M <= 4 at
        // 4096 x 11008, 8192 x 11008, 5120 x 13824, 8192 x 5120 and
        // 4096 x 15360, timed side by side.  16 waves where the rows divide
        // evenly over the grid's 4096 waves, else 8, whose 2048 waves leave a
        // smaller last round (5120 rows: 1.25 rows per wave against 2.5; 8
        // waves were 1.08-1.13x ahead there).
        if (M <= 4 && K >= 4096 && skinny_vec_fits(M, K, 4) &&
            4 * skinny_vec_npad(K, 4) <= 5LL * (K / 8)) {
            c.blocks = 1;
            c.unroll = 4;
            c.waves = N % 4096 == 0 ? 16 : 8;
            c.stages = 1;
            return c;
        }
    }
    if (lds_ok && M > 4) {
        c.blocks = small_n ? 1 : (K <= 2048 ? 2 : (K <= 4096 ? 1 : 3));
        c.unroll = 0;
        c.waves = small_n && N <= 4096 ? 16 : 8;
        c.stages = !small_n ? 2 : (N <= 4096 ? 4 : 3);
    } else {
        c.blocks = M <= 4 ? 1 : 2;
        c.unroll = M <= 4 ? 4 : 2;
        c.stages = 0;
    }
    return c;
}

bool skinny_fits(const void* A, const void* B, int M, int K)
{
    return M >= 1 && M <= kSkinnyMaxM && K % 8 == 0 && aligned(A, 16) && aligned(B, 16);
}

// M = 17 .. 64 rows of A: the LDS form only, A staged in 16-row blocks.
constexpr int kSkinnyWideMaxM = 64;
bool skinny_wide_fits(const void* A, const void* B, int M, int K)
{
    return M > kSkinnyMaxM && M <= kSkinnyWideMaxM && K > 0 && K % kSkinnyKc == 0 && aligned(A, 16) &&
           aligned(B, 16);
}

int skinny_impl(const void* A, const void* B, void* C, int M, int N, int K, const gf_skinny_cfg& cfg,
                hipStream_t stream)
{
    const int idx = find_skinny(cfg);
    if (idx < 0 || !g_skinny_table[idx]) return GF_ERR_UNSUPPORTED;
    const SkinnyDesc& d = kSkinnyConfigs[idx];
    if (d.stages == 1 && !skinny_vec_fits(M, K, d.unroll)) return GF_ERR_UNSUPPORTED;
    if (d.stages < 0 && !skinny_split_fits(M, K, d.unroll, d.waves)) return GF_ERR_UNSUPPORTED;
    if (d.stages >= 2 && (K % kSkinnyKc != 0 || K == 0)) return GF_ERR_UNSUPPORTED;
    if (M > kSkinnyMaxM && (d.stages < 2 || M > skinny_lds_max_m(d.blocks, d.stages, d.waves)))
        return GF_ERR_UNSUPPORTED;
    return launch_status(g_skinny_table[idx](static_cast<const uint16_t*>(A),
                                             static_cast<const uint16_t*>(B),
                                             static_cast<uint16_t*>(C), M, N, K, stream));
}

int find_gemv(const gf_gemv_cfg& c)
{
    for (int i = 0; i < kNumGemv; ++i) {
        const GemvDesc& d = kGemvConfigs[i];
        if (d.rows == c.rows_per_wave && d.unroll == c.unroll && d.waves == c.waves) return i;
    }
    return -1;
}

// Launch shape, from sweeps of the compiled shapes (batches of back-to-back
// calls, W rotated over more than the MALL) at N x K = 8192^2, 16384 x 8192,
// 8192 x 16384, 4096 x 8192, 16384 x 4096, 14336 x 4096, 28672 x 4096,
// 8192 x 4096, 4096^2, 4096 x 14336, 12288 x 6144 and 2048 x 8192:
//  * the split form (a workgroup's waves split K, the grid streaming one
//    band of W) where K is a multiple of 8192 and W has at least 4096 rows:
//    at K = 8192 one row per task, 4 waves with 4 chunks in flight per
//    lane, 512 workgroups (two per CU): 8192^2 20.8 us = 6.45 TB/s,
//    4096 x 8192 11.6 us, 16384 x 8192 39.6 us, 1.3-2 % ahead of two rows
//    per task on 8 waves and 256 workgroups at all three; beyond K = 8192
//    one row per task on 8 waves with 2 chunks, 256 workgroups (8192 x
//    16384: 39.1 us = 6.87 TB/s, first of the sweep);
//  * else one row per wave: 8 chunks per lane in flight and 2-wave
//    workgroups when each row splits into whole 512-chunk steps (K % 4096
//    == 0; 1-2 % ahead of 4 chunks at every such shape), else 4 chunks and
//    4-wave workgroups;
//  * smaller W: 2 chunks in flight and 1-wave workgroups from 2048^2 up,
//    below that 8 waves with 1 chunk (launch-bound).
gf_gemv_cfg default_gemv_cfg(int N, int K)
{
    gf_gemv_cfg c;
    const int64_t nk = (int64_t)N * K;
    c.blocks = 0;
    c.rows_per_wave = 1;
    if (nk >= (int64_t)4096 * 4096) {
        if (N >= 4096 && K % 8192 == 0 && K <= kGemvXldsMaxK) {
            if (K == 8192) { c.unroll = 4; c.waves = 4; c.blocks = 512; }
            else { c.unroll = 2; c.waves = 8; c.blocks = 256; }
        } else if (K % 4096 == 0) {
            c.unroll = 8; c.waves = 2;
        } else {
            c.unroll = 4; c.waves = 4;
        }
    } else if (nk >= (int64_t)2048 * 2048) {
        c.unroll = 2; c.waves = 1;
    } else {
        c.unroll = 1; c.waves = 8;
    }
    return c;
}

int gemv_impl(const void* W, const void* x, void* y, int N, int K, const gf_gemv_cfg& cfg,
              hipStream_t stream)
{
    if (N < 0 || K < 0 || (int64_t)N * K > kMaxElems || cfg.blocks < 0) return GF_ERR_INVALID_ARG;
    if (N > 0 && K > 0 && (!W || !aligned(W, 2))) return GF_ERR_INVALID_ARG;
    if (N > 0 && K > 0 && (!x || !aligned(x, 2))) return GF_ERR_INVALID_ARG;
    if (N > 0 && (!y || !aligned(y, 2))) return GF_ERR_INVALID_ARG;
    const int idx = find_gemv(cfg);
    if (idx < 0) return GF_ERR_UNSUPPORTED;
    if (N == 0) return GF_OK;
    const bool al = aligned(W, 16) && aligned(x, 16) && K % 8 == 0;
    GemvLaunchFn fn = g_gemv_table[idx][al ? 1 : 0];
    if (!fn) return GF_ERR_UNSUPPORTED;
    return launch_status(fn(static_cast<const uint16_t*>(W), static_cast<const uint16_t*>(x),
                            static_cast<uint16_t*>(y), N, K, cfg.blocks, stream));
}

}  // namespace
}  // namespace gf

using namespace gf;

extern "C" {

int gemm_f16_nt_cfg(const void* A, const void* B, void* C, int M, int N, int K,
                    const gf_gemm_cfg* cfg, void* stream)
{
    if (!cfg) return GF_ERR_INVALID_ARG;
    int rc = validate_gemm(A, B, C, M, N, K, 2);
    if (rc) return rc;
    if (find_gemm(*cfg) < 0) return GF_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return GF_OK;
    const int nkt = ceil_div(K, cfg->block_k);
    return run_gemm(A, B, C, M, N, K, *cfg, EPI_F16, 1, nkt, aligned(C, 16),
                    static_cast<hipStream_t>(stream));
}

int gemm_f16_nt(const void* A, const void* B, void* C, int M, int N, int K, void* stream)
{
    // A handful of rows of A: the skinny kernel streams B once.  From 17 to
    // 64 rows too where B has at most 8192 rows and K >= 4096: there a
    // 64-row tile grid leaves most CUs idle (128 workgroups at N = 8192), and
    // the LDS form ran 1.07-3.3x faster; from 14336 rows of B, or at
    // K = 2048, the tiles were ahead.
    auto takes_skinny = [&](const void* a, int m) {
        return skinny_fits(a, B, m, K) || (skinny_wide_fits(a, B, m, K) && N <= 8192 && K >= 4096);
    };
    if (M > 0 && N > 0 && takes_skinny(A, M)) {
        const int rc = validate_gemm(A, B, C, M, N, K, 2);
        if (rc) return rc;
        return skinny_impl(A, B, C, M, N, K, default_skinny_cfg(M, N, K),
                           static_cast<hipStream_t>(stream));
    }
    const gf_gemm_cfg cfg = default_gemm_cfg(M, N, K);
    const int m1 = row_split(M, N, cfg);
    if (m1 < M) {
        const int rc = validate_gemm(A, B, C, M, N, K, 2);
        if (rc) return rc;
        const int r1 = gemm_f16_nt_cfg(A, B, C, m1, N, K, &cfg, stream);
        if (r1) return r1;
        const char* At = static_cast<const char*>(A) + (size_t)m1 * K * 2;
        char* Ct = static_cast<char*>(C) + (size_t)m1 * N * 2;
        const int mt = M - m1;
        if (takes_skinny(At, mt))
            return skinny_impl(At, B, Ct, mt, N, K, default_skinny_cfg(mt, N, K),
                               static_cast<hipStream_t>(stream));
        const gf_gemm_cfg tail = tail_gemm_cfg(mt, N);
        return gemm_f16_nt_cfg(At, B, Ct, mt, N, K, &tail, stream);
    }
    return gemm_f16_nt_cfg(A, B, C, M, N, K, &cfg, stream);
}

int gemm_f16_nt_skinny(const void* A, const void* B, void* C, int M, int N, int K,
                       const gf_skinny_cfg* cfg, void* stream)
{
    int rc = validate_gemm(A, B, C, M, N, K, 2);
    if (rc) return rc;
    if (M == 0 || N == 0) return GF_OK;
    if (!skinny_fits(A, B, M, K) && !skinny_wide_fits(A, B, M, K)) return GF_ERR_UNSUPPORTED;
    const gf_skinny_cfg c = cfg ? *cfg : default_skinny_cfg(M, N, K);
    return skinny_impl(A, B, C, M, N, K, c, static_cast<hipStream_t>(stream));
}

int gf_skinny_config_count(void) { return kNumSkinny; }

int gf_skinny_config_get(int i, gf_skinny_cfg* out)
{
    if (!out || i < 0 || i >= kNumSkinny) return GF_ERR_INVALID_ARG;
    out->blocks = kSkinnyConfigs[i].blocks;
    out->unroll = kSkinnyConfigs[i].unroll;
    out->waves = kSkinnyConfigs[i].waves;
    out->stages = kSkinnyConfigs[i].stages;
    return GF_OK;
}

int gf_skinny_default_config(int M, int N, int K, gf_skinny_cfg* out)
{
    if (!out || M < 1 || M > kSkinnyWideMaxM || N < 0 || K < 0) return GF_ERR_INVALID_ARG;
    *out = default_skinny_cfg(M, N, K);
    return GF_OK;
}

int gemm_f16_cfg(const void* A, const void* B, void* C, int M, int N, int K, int a_kmajor,
                 int b_kmajor, const gf_gemm_cfg* cfg, void* stream)
{
    if (!cfg || (a_kmajor != 0 && a_kmajor != 1) || (b_kmajor != 0 && b_kmajor != 1))
        return GF_ERR_INVALID_ARG;
    if (a_kmajor == 0 && b_kmajor == 0) return gemm_f16_nt_cfg(A, B, C, M, N, K, cfg, stream);
    int rc = validate_gemm(A, B, C, M, N, K, 2);
    if (rc) return rc;
    const int idx = find_gemm(*cfg);
    if (idx < 0 || !has_layouts(kGemmConfigs[idx])) return GF_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return GF_OK;
    // Fast path: 16-byte aligned operands whose contiguous extent (K for a
    // K-contiguous operand, M or N for a K-major one) is a multiple of 8.
    const bool al = aligned(A, 16) && aligned(B, 16) && aligned(C, 16) &&
                    (a_kmajor ? M % 8 == 0 : K % 8 == 0) && (b_kmajor ? N % 8 == 0 : K % 8 == 0);
    GemmLaunchFn fn = g_gemm_layout_table[idx][a_kmajor * 2 + b_kmajor][al ? 1 : 0];
    if (!fn) return GF_ERR_UNSUPPORTED;
    GemmArgs a;
    a.A = static_cast<const uint16_t*>(A);
    a.B = static_cast<const uint16_t*>(B);
    a.C = C;
    a.M = M; a.N = N; a.K = K;
    a.kt_per_slice = ceil_div(K, cfg->block_k);
    a.raster = panel_of(cfg->raster);
    return launch_status(fn(a, 1, static_cast<hipStream_t>(stream)));
}

// A K-major operand runs the schedule-2 tiles (the only ones with the
// transposing fragment reads): 256 x 256 once 256 of them fill the CUs,
// else 128 x 128 with two stages, two workgroups per CU -- which is also
// 1.14-1.18x ahead of 256 x 256 for K <= 256 (8192^2 and 4096^2, NN and TN,
// timed side by side; even at K = 512, behind from K = 1024).
int gemm_f16(const void* A, const void* B, void* C, int M, int N, int K, int a_kmajor, int b_kmajor,
             void* stream)
{
    gf_gemm_cfg cfg = default_gemm_cfg(M, N, K);
    if (a_kmajor || b_kmajor) {
        const int64_t t256 = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
        cfg = t256 >= 256 && K > 256 ? make_cfg(256, 256, 64, 2, 256, 0, 2) : make_cfg(128, 128, 64, 2, 256, 0, 2);
    }
    return gemm_f16_cfg(A, B, C, M, N, K, a_kmajor, b_kmajor, &cfg, stream);
}

int gemm_f16_nn(const void* A, const void* B, void* C, int M, int N, int K, void* stream)
{
    return gemm_f16(A, B, C, M, N, K, 0, 1, stream);
}

int gemm_f16_tn(const void* A, const void* B, void* C, int M, int N, int K, void* stream)
{
    return gemm_f16(A, B, C, M, N, K, 1, 1, stream);
}

int gemm_f16_nt_splitk(const void* A, const void* B, float* C32, int M, int N, int K, int split_k,
                       void* stream)
{
    return splitk_impl(A, B, C32, M, N, K, split_k, GF_SPLITK_ATOMIC, nullptr, 0,
                       default_splitk_cfg(M, N, K, split_k, true), static_cast<hipStream_t>(stream));
}

int gemm_f16_nt_splitk_cfg(const void* A, const void* B, void* C, int M, int N, int K, int split_k,
                           int mode, void* workspace, size_t workspace_bytes, const gf_gemm_cfg* cfg,
                           void* stream)
{
    if (!cfg) return GF_ERR_INVALID_ARG;
    const int idx = find_gemm(*cfg);
    if (idx >= 0 && !kGemmConfigs[idx].core) return GF_ERR_UNSUPPORTED;   // no fp32 epilogues compiled
    if (mode == GF_SPLITK_F16)
        return splitk_f16_impl(A, B, C, M, N, K, split_k, workspace, workspace_bytes, *cfg,
                               static_cast<hipStream_t>(stream));
    return splitk_impl(A, B, static_cast<float*>(C), M, N, K, split_k, mode, workspace,
                       workspace_bytes, *cfg, static_cast<hipStream_t>(stream));
}

int gemm_f16_nt_splitk_f16(const void* A, const void* B, void* C, int M, int N, int K,
                           int split_k, void* workspace, size_t workspace_bytes, void* stream)
{
    return splitk_f16_impl(A, B, C, M, N, K, split_k, workspace, workspace_bytes,
                           default_splitk_cfg(M, N, K, split_k), static_cast<hipStream_t>(stream));
}

size_t gemm_f16_nt_splitk_workspace_bytes(int M, int N, int split_k)
{
    if (M < 0 || N < 0 || split_k < 1) return 0;
    return (size_t)split_k * (size_t)M * (size_t)N * sizeof(float);
}

int gemm_f16_nt_splitk_ex(const void* A, const void* B, float* C32, int M, int N, int K, int split_k,
                          int mode, void* workspace, size_t workspace_bytes, void* stream)
{
    return splitk_impl(A, B, C32, M, N, K, split_k, mode, workspace, workspace_bytes,
                       default_splitk_cfg(M, N, K, split_k, mode == GF_SPLITK_ATOMIC),
                       static_cast<hipStream_t>(stream));
}

int gemm_f16_nt_splitk_noalloc(const void* A, const void* B, float* C32, int M, int N, int K,
                               int split_k, void* stream)
{
    if (split_k < 1) return GF_ERR_INVALID_ARG;
    if (M < 0 || N < 0) return GF_ERR_INVALID_ARG;
    if ((uint64_t)split_k * (uint64_t)M * (uint64_t)N * sizeof(float) > kScratchBytes)
        return GF_ERR_TOO_LARGE;
    int rc = validate_gemm(A, B, C32, M, N, K, 4);
    if (rc) return rc;
    if (M == 0 || N == 0) return GF_OK;
    void* ws = nullptr;
    rc = scratch_for_stream(static_cast<hipStream_t>(stream), &ws);
    if (rc) return rc;
    return splitk_impl(A, B, C32, M, N, K, split_k, GF_SPLITK_TWOPASS, ws, kScratchBytes,
                       default_splitk_cfg(M, N, K, split_k), static_cast<hipStream_t>(stream));
}

size_t gf_noalloc_scratch_bytes(void) { return kScratchBytes; }

int gemv_f16_cfg(const void* W, const void* x, void* y, int N, int K, const gf_gemv_cfg* cfg,
                 void* stream)
{
    if (!cfg) return GF_ERR_INVALID_ARG;
    return gemv_impl(W, x, y, N, K, *cfg, static_cast<hipStream_t>(stream));
}

int gemv_f16(const void* W, const void* x, void* y, int N, int K, void* stream)
{
    const gf_gemv_cfg cfg = default_gemv_cfg(N, K);
    return gemv_impl(W, x, y, N, K, cfg, static_cast<hipStream_t>(stream));
}

int gf_gemm_config_count(void) { return kNumGemm; }

int gf_gemm_config_get(int i, gf_gemm_cfg* out)
{
    if (i < 0 || i >= kNumGemm || !out) return GF_ERR_INVALID_ARG;
    const GemmDesc& d = kGemmConfigs[i];
    *out = make_cfg(d.bm, d.bn, d.bk, d.stages, d.threads, 1, d.sched);
    // A config with no compiled kernel (illegal LDS or wave layout) is unsupported.
    return g_gemm_table[i][EPI_F16 * 2 + 1] ? GF_OK : GF_ERR_UNSUPPORTED;
}

int gf_gemv_config_count(void) { return kNumGemv; }

int gf_gemv_config_get(int i, gf_gemv_cfg* out)
{
    if (i < 0 || i >= kNumGemv || !out) return GF_ERR_INVALID_ARG;
    out->rows_per_wave = kGemvConfigs[i].rows;
    out->unroll = kGemvConfigs[i].unroll;
    out->waves = kGemvConfigs[i].waves;
    out->blocks = 0;
    return GF_OK;
}

int gf_gemm_default_config(int M, int N, int K, gf_gemm_cfg* out)
{
    if (!out || M < 0 || N < 0 || K < 0) return GF_ERR_INVALID_ARG;
    *out = default_gemm_cfg(M, N, K);
    return GF_OK;
}

int gf_gemv_default_config(int N, int K, gf_gemv_cfg* out)
{
    if (!out || N < 0 || K < 0) return GF_ERR_INVALID_ARG;
    *out = default_gemv_cfg(N, K);
    return GF_OK;
}

const char* gf_status_string(int status)
{
    switch (status) {
    case GF_OK: return "GF_OK";
    case GF_ERR_INVALID_ARG: return "GF_ERR_INVALID_ARG: invalid argument";
    case GF_ERR_HIP: return "GF_ERR_HIP: HIP runtime error at launch";
    case GF_ERR_UNSUPPORTED: return "GF_ERR_UNSUPPORTED: no compiled kernel for this config";
    case GF_ERR_TOO_LARGE:
        return "GF_ERR_TOO_LARGE: split_k * M * N * 4 bytes exceed the 64 MiB no-allocation scratch";
    default: return "unknown status";
    }
}

}  // extern "C"
