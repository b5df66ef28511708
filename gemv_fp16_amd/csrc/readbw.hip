// HBM streaming-read ceiling probe: a diagnostic program, not part of the
// library.  It reads 134,217,728 bytes per launch -- the size of the GEMV's
// W at N = K = 8192 -- with 128-bit non-temporal loads, grid-stride over the
// flat buffer (all waves together sweep one contiguous window).  "cold"
// rotates over 5 buffers (640 MiB, more than the 256 MiB MALL), "warm" reuses
// one.  Time per launch is taken from HIP events around 100 back-to-back
// launches.  Usage: ./readbw
#include <hip/hip_runtime.h>
#include <cstdio>
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <int U>
__global__ __launch_bounds__(256) void rd(const u32x4* __restrict__ p, size_t n, unsigned* out) {
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  size_t stride = (size_t)gridDim.x * 256;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= p[i];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * 4 + threadIdx.x / 64] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}
template <int U> void run(u32x4** bufs, size_t n, unsigned* out, int grid) {
  hipEvent_t a, b; (void)hipEventCreate(&a); (void)hipEventCreate(&b);
  float ms[2];
  for (int warm = 0; warm < 2; ++warm) {
    for (int w = 0; w < 10; ++w) hipLaunchKernelGGL((rd<U>), dim3(grid), dim3(256), 0, 0, bufs[warm ? 0 : w % 5], n, out);
    (void)hipEventRecord(a);
    for (int r = 0; r < 100; ++r) hipLaunchKernelGGL((rd<U>), dim3(grid), dim3(256), 0, 0, bufs[warm ? 0 : r % 5], n, out);
    (void)hipEventRecord(b); (void)hipEventSynchronize(b);
    (void)hipEventElapsedTime(&ms[warm], a, b);
  }
  printf("grid %5d U%d  cold %6.2f us %6.0f GB/s   warm %6.2f us %6.0f GB/s\n", grid, U,
         ms[0] * 10, n * 16.0 / (ms[0] / 100 * 1e-3) / 1e9, ms[1] * 10, n * 16.0 / (ms[1] / 100 * 1e-3) / 1e9);
}
int main() {
  size_t bytes = 134217728ull, n = bytes / 16;
  u32x4* bufs[5]; unsigned* out;
  for (int i = 0; i < 5; ++i) { if (hipMalloc(&bufs[i], bytes) != hipSuccess) return 1; (void)hipMemset(bufs[i], 1, bytes); }
  if (hipMalloc(&out, 1 << 22) != hipSuccess) return 1;
  int grids[] = {256, 512, 1024, 2048, 4096};
  for (int g : grids) { run<2>(bufs, n, out, g); run<4>(bufs, n, out, g); run<8>(bufs, n, out, g); }
  (void)hipDeviceSynchronize();
  return 0;
}
