// Shared device helpers for the gfx950 kernels (wave64, CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

namespace gf {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define GF_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;

// s_waitcnt immediates for gfx9: vmcnt in bits [3:0] and [15:14], expcnt in
// [6:4], lgkmcnt in [11:8].  A field at its maximum means "do not wait".
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Workgroup barrier that orders LDS traffic only: waits for this wave's own
// LDS operations, then s_barrier.  The asm clobbers keep the compiler from
// moving memory accesses across it.  Global loads in flight (including
// direct-to-LDS loads) are NOT waited for; callers wait on vmcnt themselves.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    wait_lgkmcnt0();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Compile-time loop: f(std::integral_constant<int, I>{}) for I = 0 .. N-1, so
// every index in the body is a constant (no runtime indexing of register
// arrays, no dependence on the unroller's size limits).
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for_impl<I + 1, N>(f);
    }
}

template <int N, class F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl<0, N>(f);
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Dynamic LDS above 64 KiB must be opted into, per kernel and per device:
// here on the device the launch's stream belongs to (the current device for
// the null stream), made current for the call if it is another.  `done`
// holds one bit per device id below 64 whose opt-in is made (the caller
// keeps one per kernel); host threads that race only repeat the idempotent
// call.
inline hipError_t opt_in_lds(const void* kern, int bytes, std::atomic<uint64_t>& done, hipStream_t stream)
{
    int cur = 0, dev = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    dev = cur;
    if (stream) {                       // the device the launch goes to: the stream's
        hipDevice_t d;
        e = hipStreamGetDevice(stream, &d);
        if (e != hipSuccess) return e;
        dev = (int)d;
    }
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t(1) << dev) : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (dev != cur) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess) e = e2;
    }
    if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

// Map a linear workgroup index to a logical tile index so that each XCD
// receives one contiguous run of tiles.  The hardware hands consecutive
// workgroup ids to the 8 XCDs in turn, so without the remap neighbouring
// tiles (which share operand panels) land in different L2 caches.
__device__ __forceinline__ int xcd_remap(int w, int total)
{
    constexpr int kXcd = 8;
    int q = total / kXcd, r = total % kXcd;
    int xcd = w % kXcd, local = w / kXcd;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Grouped tile order: walk `panel` tile-rows (M direction) column by column,
// then move to the next panel, so that the tiles in flight together reuse a
// few A row-panels and B column-panels from cache.
__device__ __forceinline__ void grouped_tile(int L, int tiles_m, int tiles_n, int panel,
                                             int& tm, int& tn)
{
    int per_group = panel * tiles_n;
    int group = L / per_group;
    int first_m = group * panel;
    int gsize = min(panel, tiles_m - first_m);
    int in_group = L - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// Round-to-nearest-even fp32 -> fp16 (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v)
{
    _Float16 h = (_Float16)v;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}

}  // namespace gf
