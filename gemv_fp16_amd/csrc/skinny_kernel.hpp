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
#include "gemv_kernel.hpp"

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

// ---------------------------------------------------------------------------
// LDS-staged form (K % 512 == 0): row-long loads
// ---------------------------------------------------------------------------
//
// The direct form above reads 16 rows x 64 bytes per load instruction.  Here
// every load instruction moves 1 KiB of ONE row (512 consecutive k) straight
// into LDS, the pattern the GEMV streams at: per 512-k chunk a workgroup
// loads its 16 * NB rows of B and MA rows of A, MA = 4, 8 or 16, the fewest
// that cover M (rows past M are clamped to a valid row; an MFMA row of A only
// reaches the same row of the result, and those rows are not stored, so the
// fragment reads of the 16 - MA rows that are not staged re-read row
// MA - 1).  For 17 to 64 rows MA = 32, 48 or 64: A sits in 16-row blocks,
// each of which meets every B fragment with accumulators of its own, so B
// is still read once.  Chunk c of a row sits at 16-byte slot
// c ^ (row % 16), so the 16 lanes that read one fragment (16 rows, same k)
// hit 16 different bank groups.  S chunks ring through LDS; every wave
// issues the same number of loads per chunk, so each wait is a constant.
// The 16 k-steps of a chunk are dealt to the W waves; their partial tiles
// are summed at the end as in the direct form.
constexpr int kSkinnyKc = 512;                  // k per chunk (1 KiB per row)

template <int NB, int S, int W, int MA = 16>
struct SkinnyLdsCfg {
    static constexpr int ROWS = 16 * NB + MA;           // B rows, then MA A rows
    static constexpr int CHUNK_BYTES = ROWS * kSkinnyKc * 2;
    static constexpr int LW = ROWS / W;                 // loads per wave per chunk
    static constexpr int LDS_BYTES = S * CHUNK_BYTES;
    static constexpr int MB = MA > 16 ? MA / 16 : 1;     // 16-row blocks of A
    static constexpr bool kValid =
        W <= 16 && ROWS % W == 0 && LDS_BYTES <= 160 * 1024 && S >= 2 && LW * S < 64 &&
        (MA == 4 || MA == 8 || MA == 16 || MA == 32 || MA == 48 || MA == 64);
};

template <int NB, int S, int W, int MA>
__global__ __launch_bounds__(W * kWave) void skinny_lds_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, uint16_t* __restrict__ C, int M,
    int N, int K)
{
#if defined(__HIP_DEVICE_COMPILE__)
    typedef SkinnyLdsCfg<NB, S, W, MA> Cf;
    extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
    GF_LDS char* smem = (GF_LDS char*)smem_raw;
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int n0 = blockIdx.x * NB * 16;
    const int nchunks = K / kSkinnyKc;
    __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)A, 0, (int)((uint32_t)M * (uint32_t)K * 2u), 0x00020000);
    __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)B, 0, (int)((uint32_t)N * (uint32_t)K * 2u), 0x00020000);
    // Load q of this wave covers tile row i = q * W + wave: B rows first,
    // then A.  Byte offset of the row's chunk 0 (scalar) and of the lane's
    // swizzled 16 bytes inside the chunk (vector).
    auto row_of = [&](int q) { return q * W + wave; };
    auto issue_chunk = [&](int chunk, int slot) {
#pragma unroll
        for (int q = 0; q < Cf::LW; ++q) {
            const int i = row_of(q);
            const bool is_b = i < 16 * NB;
            const int grow = is_b ? min(n0 + i, N - 1) : min(i - 16 * NB, M - 1);
            const uint32_t soff = ((uint32_t)grow * (uint32_t)K + (uint32_t)chunk * kSkinnyKc) * 2u;
            const uint32_t voff = (uint32_t)((lane ^ (i % 16)) * 16);
            GF_LDS char* dst = smem + slot * Cf::CHUNK_BYTES + i * (kSkinnyKc * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_b ? rb : ra, (GF_LDS void*)dst, 16, voff, soff, 0, 0);
        }
    };
    // Fragment of tile row block `blk` (16 rows) at k-step ks of a chunk:
    // lane l reads row 16 * blk + l % 16, 16-byte chunk 4 * ks + l / 16.
    const int r16 = lane % 16, kq = lane / 16;
    auto frag = [&](int slot, int blk, int ks) {
        const int rr = (blk == NB && MA < 16) ? min(r16, MA - 1) : r16;   // row within the 16-row block
        const int row = 16 * blk + rr;
        const int c = (4 * ks + kq) ^ rr;
        return *(const GF_LDS half8*)(smem + slot * Cf::CHUNK_BYTES + row * (kSkinnyKc * 2) + c * 16);
    };
    constexpr int MB = Cf::MB;
    floatx4 acc[MB][NB];
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[b][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    // Prologue: chunks 0 .. S-2 (chunk indices past the end load a valid
    // chunk 0 again, keeping the count of loads in flight fixed).
#pragma unroll
    for (int t = 0; t < S - 1; ++t) issue_chunk(t < nchunks ? t : 0, t);
    for (int t = 0; t < nchunks; ++t) {
        wait_vmcnt<Cf::LW * (S - 2)>();          // this wave's loads of chunk t landed
        lds_barrier();                           // everyone's; chunk t - 1's slot is free
        const int tn = t + S - 1;
        issue_chunk(tn < nchunks ? tn : 0, tn % S);
        const int slot = t % S;
#pragma unroll
        for (int ks = 0; ks < kSkinnyKc / 32; ++ks) {
            if (ks % W != wave % W) continue;    // wave-uniform
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                const half8 a = frag(slot, NB + b, ks);
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    acc[b][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, frag(slot, j, ks), acc[b][j], 0, 0, 0);
            }
        }
    }
    wait_vmcnt<0>();
    lds_barrier();                               // stage memory is free: reuse it for the partials
    floatx4* part = (floatx4*)smem_raw;         // [W][MB * NB][64]
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int j = 0; j < NB; ++j) part[((wave * MB + b) * NB + j) * kWave + lane] = acc[b][j];
    __syncthreads();
    static_assert(MB * NB <= W, "one thread per partial tile lane");
    if (threadIdx.x < MB * NB * kWave) {
        const int bj = threadIdx.x / kWave, l = threadIdx.x % kWave;   // bj = b * NB + j
        const int b = bj / NB, j = bj % NB;
        floatx4 sum = part[bj * kWave + l];
#pragma unroll
        for (int w = 1; w < W; ++w) sum += part[(w * MB * NB + bj) * kWave + l];
        const int n = n0 + j * 16 + l % 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * b + 4 * (l / 16) + i;
            if (m < M && n < N) C[(size_t)m * N + n] = f32_to_f16_bits(sum[i]);
        }
    }
#endif
}

template <int NB, int S, int W, int MA>
hipError_t launch_skinny_lds_ma(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                                hipStream_t stream)
{
    typedef SkinnyLdsCfg<NB, S, W, MA> Cf;
    static_assert(Cf::kValid, "skinny LDS config");
    auto kern = skinny_lds_kernel<NB, S, W, MA>;
    static std::atomic<uint64_t> lds_opt_in{0};   // devices where the LDS size is opted into
    {
        const hipError_t e = opt_in_lds((const void*)kern, Cf::LDS_BYTES, lds_opt_in, stream);
        if (e != hipSuccess) return e;
    }
    const int grid = ceil_div(N, NB * 16);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(W * kWave), Cf::LDS_BYTES, stream, A, B, C, M, N, K);
    return hipGetLastError();
}

// The LDS-staged launch for M rows of A: the fewest staged A rows (4, 8, 16,
// or 32, 48, 64 in 16-row blocks) that cover M and divide evenly over the
// waves.  M past what the config's LDS holds (skinny_lds_max_m) returns
// hipErrorInvalidValue; callers check it first.
template <int NB, int S, int W>
hipError_t launch_skinny_lds(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                             hipStream_t stream)
{
    static_assert(SkinnyLdsCfg<NB, S, W, 16>::kValid, "skinny LDS config");
    if constexpr (SkinnyLdsCfg<NB, S, W, 4>::kValid)
        if (M <= 4) return launch_skinny_lds_ma<NB, S, W, 4>(A, B, C, M, N, K, stream);
    if constexpr (SkinnyLdsCfg<NB, S, W, 8>::kValid)
        if (M <= 8) return launch_skinny_lds_ma<NB, S, W, 8>(A, B, C, M, N, K, stream);
    if (M <= 16) return launch_skinny_lds_ma<NB, S, W, 16>(A, B, C, M, N, K, stream);
    if constexpr (SkinnyLdsCfg<NB, S, W, 32>::kValid)
        if (M <= 32) return launch_skinny_lds_ma<NB, S, W, 32>(A, B, C, M, N, K, stream);
    if constexpr (SkinnyLdsCfg<NB, S, W, 48>::kValid)
        if (M <= 48) return launch_skinny_lds_ma<NB, S, W, 48>(A, B, C, M, N, K, stream);
    if constexpr (SkinnyLdsCfg<NB, S, W, 64>::kValid)
        if (M <= 64) return launch_skinny_lds_ma<NB, S, W, 64>(A, B, C, M, N, K, stream);
    return hipErrorInvalidValue;
}

// The most rows of A the LDS form of (NB, S, W) takes: 16, or the largest of
// 32, 48, 64 up to which every block count fits (the launch above).
constexpr int skinny_lds_max_m(int NB, int S, int W)
{
    int best = 16;
    for (int ma = 32; ma <= 64; ma += 16) {
        const int rows = 16 * NB + ma;
        if (!(rows % W == 0 && S * rows * kSkinnyKc * 2 <= 160 * 1024 && (rows / W) * S < 64)) break;
        best = ma;
    }
    return best;
}

// ---------------------------------------------------------------------------
// Vector form (M <= 8): the GEMV's access pattern, M vectors at once
// ---------------------------------------------------------------------------
//
// Both MFMA forms above pay for the matrix cores' operand layout: the direct
// form reads 16 rows x 64 bytes of B per load instruction, the LDS form a
// barrier per 512-k chunk.  For a handful of rows of A, B is streamed here
// exactly as the GEMV streams W: a wave owns ROWS consecutive rows of B, its
// 64 lanes split K (lane l takes the 16-byte chunks l, l + 64, ... of each
// row, UNROLL per row per step, the next step's loads in flight while this
// one is multiplied), non-temporal 128-bit loads straight into registers.
// The M <= MV rows of A are staged once per workgroup in LDS (MV * K * 2
// bytes, rows past M zero), after the wave's first loads of B are issued; each
// chunk of B meets the M matching chunks of A in v_dot2_f32_f16 (fp32
// accumulation).  When a wave finishes its rows it folds each of its ROWS x MV
// sums across the lanes with DPP and writes the fp16 results.  One workgroup
// per CU walks the row groups grid-stride, so A is staged once per CU.  As
// in the GEMV's split form, the loads of the next task are issued
// unconditionally in the steady-state loop (a load under a branch would make
// the compiler wait for every load in flight, the next task's included,
// before each multiply).  When K / 8 is not a multiple of STEP the last
// step of a row runs past its end: those lanes load a chunk of the row that
// exists and multiply zeros instead (A is staged with its rows padded by zero
// chunks to a whole number of steps, and the B chunk is replaced by zeros,
// so that an infinite B entry cannot turn the padding into a NaN).
// Requires K % 8 == 0 and MV * (K / 8 rounded up to STEP) * 16 <= 160 KiB.
template <int MV, int ROWS, int UNROLL, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void skinny_vec_kernel(const uint16_t* __restrict__ A,
                                                                const uint16_t* __restrict__ B,
                                                                uint16_t* __restrict__ C, int M, int N, int K)
{
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(ROWS * MV <= kWave, "one lane stores each result");
    extern __shared__ __attribute__((aligned(16))) char vec_smem[];
    half8* as = (half8*)vec_smem;                      // [MV][npad]
    constexpr int STEP = kWave * UNROLL;               // chunks of a row per step
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int nch = K / 8;
    const int spg = ceil_div(nch, STEP);               // steps per row group
    const int npad = spg * STEP;                       // A's row length in LDS, zero-padded
    const bool ragged = npad != nch;
    const int groups = ceil_div(N, ROWS);
    const int g0 = blockIdx.x * WAVES + wave, gstride = gridDim.x * WAVES;
    const int my_groups = g0 < groups ? (groups - g0 + gstride - 1) / gstride : 0;
    const int ntasks = my_groups * spg;
    const half8* Bv = (const half8*)B;

    half8 buf[2][ROWS][UNROLL];
    auto load = [&](int i, half8 (&b)[ROWS][UNROLL]) __attribute__((always_inline)) {
        const int g = g0 + (i / spg) * gstride;
        const int c0 = (i % spg) * STEP + lane;
#pragma unroll
        for (int r = 0; r < ROWS; ++r) {
            const half8* wr = Bv + (size_t)min(g * ROWS + r, N - 1) * nch;
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
                b[r][u] = __builtin_nontemporal_load(wr + min(c0 + u * kWave, nch - 1));
        }
    };
    if (ntasks > 0) load(0, buf[0]);                   // B traffic starts before A is staged
    const half8* Av = (const half8*)A;
    for (int j = threadIdx.x; j < MV * npad; j += WAVES * kWave) {
        const int m = j / npad, c = j - m * npad;
        as[j] = m < M && c < nch ? Av[(size_t)m * nch + c] : half8{};
    }
    __syncthreads();

    float acc[ROWS][MV];
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
        for (int m = 0; m < MV; ++m) acc[r][m] = 0.0f;
    auto compute = [&](int i, half8 (&b)[ROWS][UNROLL]) __attribute__((always_inline)) {
        const int c0 = (i % spg) * STEP + lane;
        if (ragged && i % spg == spg - 1) {            // wave-uniform: a row's last step
#pragma unroll
            for (int u = 0; u < UNROLL; ++u)
#pragma unroll
                for (int r = 0; r < ROWS; ++r)
                    if (c0 + u * kWave >= nch) b[r][u] = half8{};
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int m = 0; m < MV; ++m) {
                const half8 xv = as[m * npad + c0 + u * kWave];
#pragma unroll
                for (int r = 0; r < ROWS; ++r) acc[r][m] = dot8(b[r][u], xv, acc[r][m]);
            }
        if (i % spg == spg - 1) {                      // the wave's rows are done
            const int row0 = (g0 + (i / spg) * gstride) * ROWS;
#pragma unroll
            for (int r = 0; r < ROWS; ++r)
#pragma unroll
                for (int m = 0; m < MV; ++m) {
                    const float sum = wave_sum(acc[r][m]);
                    if (lane == r * MV + m && m < M && row0 + r < N)
                        C[(size_t)m * N + row0 + r] = f32_to_f16_bits(sum);
                    acc[r][m] = 0.0f;
                }
        }
    };
    int i = 0;
    for (; i + 2 < ntasks; i += 2) {                   // tasks i + 1 and i + 2 exist
        load(i + 1, buf[1]);
        __builtin_amdgcn_sched_barrier(0);             // the loads leave before the multiply waits
        compute(i, buf[0]);
        load(i + 2, buf[0]);
        __builtin_amdgcn_sched_barrier(0);
        compute(i + 1, buf[1]);
    }
    if (i + 1 < ntasks) {
        load(i + 1, buf[1]);
        compute(i, buf[0]);
        compute(i + 1, buf[1]);
    } else if (i < ntasks) {
        compute(i, buf[0]);
    }
#endif
}

constexpr int kSkinnyVecMaxM = 8;
constexpr int kSkinnyVecGrid = 256;                    // one workgroup per CU

// A-row capacity of the vector form for M rows: 1, 2, 4 or 8.
__host__ __device__ constexpr int skinny_vec_mv(int M) { return M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8)); }

// Chunks of 8 per row of A in the vector form's LDS: K / 8 rounded up to a
// whole number of 64 * unroll-chunk steps.
__host__ __device__ constexpr long long skinny_vec_npad(int K, int unroll)
{
    return ((long long)K / 8 + 64LL * unroll - 1) / (64LL * unroll) * (64LL * unroll);
}

// Whether the vector form with `unroll` runs M x K.
__host__ __device__ constexpr bool skinny_vec_fits(int M, int K, int unroll)
{
    return M >= 1 && M <= kSkinnyVecMaxM && K > 0 && K % 8 == 0 && unroll > 0 &&
           (long long)skinny_vec_mv(M) * skinny_vec_npad(K, unroll) * 16 <= 160 * 1024;
}

// Whether its rows split into whole steps (the case the default rule was
// measured on).
__host__ __device__ constexpr bool skinny_vec_whole(int K, int unroll) { return K % (512 * unroll) == 0; }

template <int MV, int ROWS, int UNROLL, int WAVES>
hipError_t launch_skinny_vec_mv(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                                hipStream_t stream)
{
    auto kern = skinny_vec_kernel<MV, ROWS, UNROLL, WAVES>;
    static std::atomic<uint64_t> lds_opt_in{0};   // devices where the LDS size is opted into
    {
        const hipError_t e = opt_in_lds((const void*)kern, 160 * 1024, lds_opt_in, stream);
        if (e != hipSuccess) return e;
    }
    const int groups = ceil_div(N, ROWS);
    int grid = ceil_div(groups, WAVES);
    if (grid > kSkinnyVecGrid) grid = kSkinnyVecGrid;
    const size_t lds = (size_t)MV * skinny_vec_npad(K, UNROLL) * 16;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(WAVES * kWave), lds, stream, A, B, C, M, N, K);
    return hipGetLastError();
}

// The vector-form launch for M rows; the caller has checked skinny_vec_fits.
template <int ROWS, int UNROLL, int WAVES>
hipError_t launch_skinny_vec(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                             hipStream_t stream)
{
    switch (skinny_vec_mv(M)) {
    case 1: return launch_skinny_vec_mv<1, ROWS, UNROLL, WAVES>(A, B, C, M, N, K, stream);
    case 2: return launch_skinny_vec_mv<2, ROWS, UNROLL, WAVES>(A, B, C, M, N, K, stream);
    case 4: return launch_skinny_vec_mv<4, ROWS, UNROLL, WAVES>(A, B, C, M, N, K, stream);
    default: return launch_skinny_vec_mv<8, ROWS, UNROLL, WAVES>(A, B, C, M, N, K, stream);
    }
}

// ---------------------------------------------------------------------------
// Split form (M <= 8, K == 512 * UNROLL * WAVES): the GEMV's split form, M
// vectors at once
// ---------------------------------------------------------------------------
//
// The GEMV's fastest launch shape lets the waves of a workgroup split K and
// the workgroups walk whole rows grid-stride, so that all of them together
// read one band of rows at a time, the order HBM serves best.  Here the same
// for up to 8 rows of A: wave w of a workgroup owns chunks [w * STEP,
// (w + 1) * STEP) of every row of B, STEP = 64 * UNROLL (lane l the chunks
// w * STEP + l + 64 u), and since K is exactly WAVES * STEP chunks of 8, a
// lane meets the same M x UNROLL chunks of A in every row: they are loaded
// once into registers, so the multiply reads nothing from LDS.  A task is
// one row of B; the next row's loads are issued before the current one is
// multiplied.  Per row, every lane's MV partial sums are folded across its
// 16-lane DPP row; the 4 row leaders of each wave park them in LDS (slots
// alternating between tasks), and after the task's one barrier thread q < MV
// adds the 4 * WAVES partials of output m = q in a fixed order and writes
// C[m][row] (deterministic).  Requires 16-byte aligned A and B.
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]: pairs
    v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]: quads
    v += dpp_f32<0x141>(v);   // row_half_mirror: 8 lanes
    v += dpp_f32<0x140>(v);   // row_mirror: every lane holds its 16-lane row's sum
    return v;
}

template <int MV, int UNROLL, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void skinny_split_kernel(const uint16_t* __restrict__ A,
                                                                  const uint16_t* __restrict__ B,
                                                                  uint16_t* __restrict__ C, int M, int N,
                                                                  int K)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int STEP = kWave * UNROLL;               // chunks of a row per wave
    constexpr int NP = 4 * WAVES;                      // partial sums per output
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    extern __shared__ __attribute__((aligned(16))) char split_smem[];
    GF_LDS float* red = (GF_LDS float*)split_smem;     // [2][MV][NP]
    const int nch = K / 8;                             // == WAVES * STEP
    const int cbase = wave * STEP + lane;
    const int ntasks = (int)blockIdx.x < N ? (N - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    if (ntasks == 0) return;                           // no rows for this workgroup
    const half8* Bv = (const half8*)B;
    auto load = [&](int i, half8 (&b)[UNROLL]) __attribute__((always_inline)) {
        const half8* wr = Bv + (size_t)(blockIdx.x + i * gridDim.x) * nch + cbase;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) b[u] = __builtin_nontemporal_load(wr + u * kWave);
    };
    half8 buf0[UNROLL], buf1[UNROLL];
    load(0, buf0);                                     // B traffic starts before A is fetched
    half8 av[MV][UNROLL];
    const half8* Av = (const half8*)A;
#pragma unroll
    for (int m = 0; m < MV; ++m)
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) av[m][u] = m < M ? Av[(size_t)m * nch + cbase + u * kWave] : half8{};
    float acc[MV];
#pragma unroll
    for (int m = 0; m < MV; ++m) acc[m] = 0.0f;
    auto compute = [&](int i, const half8 (&b)[UNROLL]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int m = 0; m < MV; ++m) acc[m] = dot8(b[u], av[m][u], acc[m]);
        GF_LDS float* slot = red + (i & 1) * MV * NP;
#pragma unroll
        for (int m = 0; m < MV; ++m) {
            const float s = row16_sum(acc[m]);
            if (lane % 16 == 0) slot[m * NP + wave * 4 + lane / 16] = s;
            acc[m] = 0.0f;
        }
        lds_barrier();
        if (threadIdx.x < MV) {
            const int m = threadIdx.x;
            float t = 0.0f;
#pragma unroll
            for (int p = 0; p < NP; ++p) t += slot[m * NP + p];
            if (m < M) C[(size_t)m * N + blockIdx.x + i * gridDim.x] = f32_to_f16_bits(t);
        }
    };
    // Steady state: the loads of tasks i + 1 and i + 2 are issued with no
    // branch around them, so each multiply waits only for its own row.
    int i = 0;
    for (; i + 2 < ntasks; i += 2) {                   // tasks i + 1 and i + 2 exist
        load(i + 1, buf1);
        __builtin_amdgcn_sched_barrier(0);             // the loads leave before the multiply waits
        compute(i, buf0);
        load(i + 2, buf0);
        __builtin_amdgcn_sched_barrier(0);
        compute(i + 1, buf1);
    }
    if (i + 1 < ntasks) {
        load(i + 1, buf1);
        compute(i, buf0);
        compute(i + 1, buf1);
    } else if (i < ntasks) {
        compute(i, buf0);
    }
#endif
}

constexpr int kSkinnySplitMaxM = 8;

// Whether the split form with `unroll` chunks and `waves` waves runs M x K.
__host__ __device__ constexpr bool skinny_split_fits(int M, int K, int unroll, int waves)
{
    return M >= 1 && M <= kSkinnySplitMaxM && unroll > 0 && waves > 0 && K == 512 * unroll * waves;
}

template <int MV, int BLOCKS, int UNROLL, int WAVES>
hipError_t launch_skinny_split_mv(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                                  hipStream_t stream)
{
    const int grid = N < BLOCKS ? N : BLOCKS;
    hipLaunchKernelGGL((skinny_split_kernel<MV, UNROLL, WAVES>), dim3(grid), dim3(WAVES * kWave),
                       (size_t)2 * MV * 4 * WAVES * 4, stream, A, B, C, M, N, K);
    return hipGetLastError();
}

// The split-form launch for M rows (BLOCKS = workgroups at most); the caller
// has checked skinny_split_fits.
template <int BLOCKS, int UNROLL, int WAVES>
hipError_t launch_skinny_split(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                               hipStream_t stream)
{
    switch (skinny_vec_mv(M)) {
    case 1: return launch_skinny_split_mv<1, BLOCKS, UNROLL, WAVES>(A, B, C, M, N, K, stream);
    case 2: return launch_skinny_split_mv<2, BLOCKS, UNROLL, WAVES>(A, B, C, M, N, K, stream);
    case 4: return launch_skinny_split_mv<4, BLOCKS, UNROLL, WAVES>(A, B, C, M, N, K, stream);
    default: return launch_skinny_split_mv<8, BLOCKS, UNROLL, WAVES>(A, B, C, M, N, K, stream);
    }
}

}  // namespace gf

