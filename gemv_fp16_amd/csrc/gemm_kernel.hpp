// Tiled fp16 NT GEMM for gfx950: C = A . B^T with fp32 MFMA accumulation.
//
// Structure (TileLang FP16 matmul autotune benchmark page, section 2: block
// tiles of block_M x block_N, a K loop over block_K tiles that is software
// pipelined over num_stages shared-memory buffers, a block-level tensor-core
// product with transpose_B, a swizzled block order for L2 reuse, and an
// epilogue that goes through shared memory) re-designed for CDNA4:
//
//  * Operand staging: both A (M x K) and B (N x K) are K-contiguous, so each
//    16-byte chunk of 8 fp16 along K is one unit.  Chunks move global -> LDS
//    with gfx950's direct-to-LDS 128-bit loads (global_load_lds_dwordx4), so
//    no VGPRs or ds_write instructions are spent on staging.  A direct-to-LDS
//    wave instruction writes 64 consecutive 16-byte LDS slots; the LDS layout
//    swizzle is applied by choosing which global chunk each lane fetches.
//  * LDS layout: per stage, A tile [BM][BK] then B tile [BN][BK], fp16,
//    rows of BK/8 chunks; chunk c of row r sits at slot c ^ swz(r).  swz
//    spreads the 8 rows read together by one MFMA operand fetch over eight
//    different 16-byte bank groups.
//  * Pipeline: STAGES LDS buffers in a ring; STAGES-1 tiles are in flight
//    while one is consumed; one workgroup barrier per K tile.
//  * Contraction: waves form a WM x WN grid over the tile; each wave owns a
//    (BM/WM) x (BN/WN) sub-tile of v_mfma_f32_32x32x16_f16 (or 16x16x32 for
//    narrow sub-tiles) accumulators.
//  * Workgroup order: optional XCD-aware remap plus grouped (panel) order.
//  * Epilogues: fp16 C through a per-wave LDS transpose and 128-bit stores;
//    fp32 atomic add (split-K); fp32 plain stores into a slice workspace
//    (deterministic two-pass split-K).
#pragma once
#include "common.hpp"

namespace gf {

enum Epi { EPI_F16 = 0, EPI_F32_ATOMIC = 1, EPI_F32_STORE = 2 };

struct GemmArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;            // fp16 C, fp32 C32, or the fp32 slice workspace
    int M, N, K;
    int kt_per_slice;   // K tiles per split-K slice (gridDim.y slices)
    int raster;         // 0: plain tile order; > 0: XCD remap + panel of this many rows
};

// 16 zero bytes: the source of direct-to-LDS chunks that lie beyond K.
static __device__ __attribute__((aligned(16))) uint32_t g_zero16[4] = {0u, 0u, 0u, 0u};

template <int BM_, int BN_, int BK_, int STAGES_, int NT_>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, NT = NT_;
    static constexpr int NWAVES = NT / kWave;
    // Square-ish wave grid; the longer tile side gets more waves.
    static constexpr int WM = (NWAVES == 4) ? 2 : (NWAVES == 8 ? (BM > BN ? 4 : 2) : 1);
    static constexpr int WN = NWAVES / WM;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MT = (WTM % 32 == 0 && WTN % 32 == 0) ? 32 : 16;  // MFMA tile
    static constexpr int KS = (MT == 32) ? 16 : 32;                          // MFMA K
    static constexpr int FM = WTM / MT, FN = WTN / MT;
    static constexpr int CH = BK / 8;                        // 16-byte chunks per row
    static constexpr int ROWS_PER_SWZ = 8 / CH;              // rows sharing one swizzle key
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LPS = (BM + BN) * CH / NT;          // 16-byte loads per thread per stage
    static constexpr int EPAD = 8;                           // fp16 pad per epilogue row
    static constexpr int EPI_BYTES = NWAVES * WTM * (WTN + EPAD) * 2;
    static constexpr int MAIN_BYTES = STAGES * STAGE_BYTES;
    static constexpr int LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;

    // A config is legal when it maps onto wave64 MFMA tiles, splits evenly
    // over the loader, and fits one CU's 160 KiB of LDS.
    static constexpr bool kValid =
        (NWAVES == 4 || NWAVES == 8) && WTM % MT == 0 && WTN % MT == 0 && WTM >= 16 &&
        WTN >= 16 && BK % KS == 0 && (CH == 4 || CH == 8) && ((BM + BN) * CH) % NT == 0 &&
        (BM * CH) % kWave == 0 && STAGES >= 1 && STAGES <= 4 && LDS_BYTES <= 160 * 1024 &&
        LPS * (STAGES > 2 ? STAGES - 2 : 0) < 64 && (WTM * (WTN / 8)) % kWave == 0;
};

__device__ __forceinline__ int swz_key(int row, int rows_per_key, int ch)
{
    return (row / rows_per_key) % ch;
}

// ---------------------------------------------------------------------------
// Operand staging
// ---------------------------------------------------------------------------

// Issue the direct-to-LDS loads of one K tile into one stage buffer.
// MASK_K: chunks with k >= K read the zero chunk instead (last, ragged tile).
template <class Cfg, bool MASK_K>
__device__ __forceinline__ void issue_tile_dma(const GemmArgs& a, GF_LDS char* stage, int m0,
                                               int n0, int k0, int tid, int wave)
{
#pragma unroll
    for (int r = 0; r < Cfg::LPS; ++r) {
        const int slot = r * Cfg::NT + tid;            // LDS slot this lane fills
        const int wslot = r * Cfg::NT + wave * kWave;  // first slot of this wave instruction
        const bool is_a = wslot < Cfg::BM * Cfg::CH;   // wave-uniform
        const int s = is_a ? slot : slot - Cfg::BM * Cfg::CH;
        const int row = s / Cfg::CH;
        const int c = (s % Cfg::CH) ^ swz_key(row, Cfg::ROWS_PER_SWZ, Cfg::CH);
        const int grow = is_a ? min(m0 + row, a.M - 1) : min(n0 + row, a.N - 1);
        const uint16_t* base = is_a ? a.A : a.B;
        const int kk = k0 + c * 8;
        const void* src = base + (size_t)grow * a.K + kk;
        if (MASK_K && kk >= a.K) src = (const void*)g_zero16;
        __builtin_amdgcn_global_load_lds(src, (GF_LDS void*)(stage + wslot * 16), 16, 0, 0);
    }
}

// Masked staging through registers for operands that are not 16-byte
// aligned or whose K is not a multiple of 8: element loads with bounds
// checks, zero fill, then one 16-byte LDS write per chunk.
template <class Cfg>
__device__ __forceinline__ void load_tile_masked(const GemmArgs& a, GF_LDS char* stage, int m0,
                                                 int n0, int k0, int tid)
{
#pragma unroll
    for (int r = 0; r < Cfg::LPS; ++r) {
        const int slot = r * Cfg::NT + tid;
        const bool is_a = slot < Cfg::BM * Cfg::CH;
        const int s = is_a ? slot : slot - Cfg::BM * Cfg::CH;
        const int row = s / Cfg::CH;
        const int c = (s % Cfg::CH) ^ swz_key(row, Cfg::ROWS_PER_SWZ, Cfg::CH);
        const int grow = is_a ? m0 + row : n0 + row;
        const int rows = is_a ? a.M : a.N;
        const uint16_t* base = is_a ? a.A : a.B;
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kk = k0 + c * 8 + e;
            v[e] = (grow < rows && kk < a.K) ? base[(size_t)grow * a.K + kk] : (uint16_t)0;
        }
        u32x4 w;
        w.x = v[0] | ((uint32_t)v[1] << 16);
        w.y = v[2] | ((uint32_t)v[3] << 16);
        w.z = v[4] | ((uint32_t)v[5] << 16);
        w.w = v[6] | ((uint32_t)v[7] << 16);
        *(GF_LDS u32x4*)(stage + slot * 16) = w;
    }
}

// ---------------------------------------------------------------------------
// MFMA over one staged K tile
// ---------------------------------------------------------------------------

template <int MT>
struct Mfma;

template <>
struct Mfma<32> {
    typedef floatx16 acc_t;
    static constexpr int NACC = 16;
    static __device__ __forceinline__ acc_t run(half8 a, half8 b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    // Output row (within the 32 x 32 block) of accumulator i in lane l;
    // the column is l % 32.
    static __device__ __forceinline__ int row(int i, int lane)
    {
        return 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
    }
};

template <>
struct Mfma<16> {
    typedef floatx4 acc_t;
    static constexpr int NACC = 4;
    static __device__ __forceinline__ acc_t run(half8 a, half8 b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int i, int lane) { return 4 * (lane / 16) + i; }
};

template <class Cfg>
__device__ __forceinline__ void compute_tile(const GF_LDS char* stage, int wm, int wn, int lane,
                                             typename Mfma<Cfg::MT>::acc_t (&acc)[Cfg::FM][Cfg::FN])
{
    constexpr int MT = Cfg::MT;
    const int lrow = lane % MT;      // operand row (A) / column (B) this lane feeds
    const int lk = lane / MT;        // which 8-element K group of the MFMA step
    const int key = swz_key(lrow, Cfg::ROWS_PER_SWZ, Cfg::CH);
    const GF_LDS char* As = stage + (wm * Cfg::WTM + lrow) * (Cfg::BK * 2);
    const GF_LDS char* Bs = stage + Cfg::A_BYTES + (wn * Cfg::WTN + lrow) * (Cfg::BK * 2);
#pragma unroll
    for (int ks = 0; ks < Cfg::BK / Cfg::KS; ++ks) {
        const int chunk = ks * (Cfg::KS / 8) + lk;
        const int off = ((chunk ^ key) * 16);
        half8 af[Cfg::FM], bf[Cfg::FN];
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
            af[fm] = *(const GF_LDS half8*)(As + fm * MT * (Cfg::BK * 2) + off);
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn)
            bf[fn] = *(const GF_LDS half8*)(Bs + fn * MT * (Cfg::BK * 2) + off);
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Cfg::FN; ++fn)
                acc[fm][fn] = Mfma<MT>::run(af[fm], bf[fn], acc[fm][fn]);
    }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <class Cfg, int EPI, bool ALIGNED>
__global__ __launch_bounds__(Cfg::NT) void gemm_nt_kernel(GemmArgs a)
{
    typedef Mfma<Cfg::MT> MF;
    typedef typename MF::acc_t acc_t;
    extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
    GF_LDS char* smem = (GF_LDS char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

    // ---- which tile ----
    const int tiles_m = ceil_div(a.M, Cfg::BM), tiles_n = ceil_div(a.N, Cfg::BN);
    int tm, tn;
    const int w = blockIdx.x;
    if (a.raster > 0) {
        grouped_tile(xcd_remap(w, tiles_m * tiles_n), tiles_m, tiles_n, a.raster, tm, tn);
    } else {
        tm = w / tiles_n;
        tn = w % tiles_n;
    }
    const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;

    // ---- which K tiles (split-K slice = blockIdx.y) ----
    const int nkt_total = ceil_div(a.K, Cfg::BK);
    const int kt_begin = blockIdx.y * a.kt_per_slice;
    const int kt_end = min(nkt_total, kt_begin + a.kt_per_slice);
    const int nk = max(0, kt_end - kt_begin);

    acc_t acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn)
#pragma unroll
            for (int i = 0; i < MF::NACC; ++i) acc[fm][fn][i] = 0.0f;

    auto stage_ptr = [&](int s) { return smem + s * Cfg::STAGE_BYTES; };
    auto issue = [&](int s, int kt) {
        const int k0 = (kt_begin + kt) * Cfg::BK;
        if constexpr (ALIGNED) {
            if (k0 + Cfg::BK <= a.K)
                issue_tile_dma<Cfg, false>(a, stage_ptr(s), m0, n0, k0, tid, wave);
            else
                issue_tile_dma<Cfg, true>(a, stage_ptr(s), m0, n0, k0, tid, wave);
        } else {
            load_tile_masked<Cfg>(a, stage_ptr(s), m0, n0, k0, tid);
        }
    };

    if constexpr (Cfg::STAGES == 1) {
        for (int kt = 0; kt < nk; ++kt) {
            lds_barrier();                       // everyone is done with the buffer
            issue(0, kt);
            wait_vmcnt<0>();
            lds_barrier();
            compute_tile<Cfg>(stage_ptr(0), wm, wn, lane, acc);
        }
    } else {
#pragma unroll
        for (int s = 0; s < Cfg::STAGES - 1; ++s)
            if (s < nk) issue(s, s);
        for (int kt = 0; kt < nk; ++kt) {
            // Tile kt has landed once at most STAGES-2 younger tiles are pending.
            if (kt + Cfg::STAGES - 2 < nk)
                wait_vmcnt<Cfg::LPS * (Cfg::STAGES - 2)>();
            else
                wait_vmcnt<0>();
            lds_barrier();                       // tile kt visible; tile kt-1 consumed
            if (kt + Cfg::STAGES - 1 < nk)
                issue((kt + Cfg::STAGES - 1) % Cfg::STAGES, kt + Cfg::STAGES - 1);
            compute_tile<Cfg>(stage_ptr(kt % Cfg::STAGES), wm, wn, lane, acc);
        }
    }

    // ---- epilogue ----
    const int wrow0 = m0 + wm * Cfg::WTM, wcol0 = n0 + wn * Cfg::WTN;
    constexpr int MT = Cfg::MT;

    if constexpr (EPI == EPI_F16) {
        uint16_t* C = (uint16_t*)a.C;
        lds_barrier();                           // operand buffers are free now
        constexpr int LDW = Cfg::WTN + Cfg::EPAD;  // fp16 per LDS row
        GF_LDS uint16_t* reg = (GF_LDS uint16_t*)(smem + wave * (Cfg::WTM * LDW * 2));
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Cfg::FN; ++fn)
#pragma unroll
                for (int i = 0; i < MF::NACC; ++i) {
                    const int r = fm * MT + MF::row(i, lane);
                    const int c = fn * MT + lane % MT;
                    reg[r * LDW + c] = f32_to_f16_bits(acc[fm][fn][i]);
                }
        asm volatile("" ::: "memory");
        wait_lgkmcnt0();
        constexpr int CPR = Cfg::WTN / 8;        // 16-byte chunks per sub-tile row
        constexpr int ITERS = Cfg::WTM * CPR / kWave;
        const bool vec_ok = ALIGNED && (a.N % 8 == 0);
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int q = it * kWave + lane;
            const int r = q / CPR, cc = q % CPR;
            const u32x4 v = *(const GF_LDS u32x4*)(reg + r * LDW + cc * 8);
            const int grow = wrow0 + r, gcol = wcol0 + cc * 8;
            if (grow >= a.M) continue;
            if (vec_ok && gcol + 8 <= a.N) {
                *(u32x4*)(C + (size_t)grow * a.N + gcol) = v;
            } else {
                const uint32_t parts[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (gcol + e < a.N)
                        C[(size_t)grow * a.N + gcol + e] = (uint16_t)(parts[e / 2] >> (16 * (e % 2)));
            }
        }
    } else if constexpr (EPI == EPI_F32_ATOMIC) {
        if (nk == 0) return;                     // an empty slice adds nothing
        float* C = (float*)a.C;
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Cfg::FN; ++fn)
#pragma unroll
                for (int i = 0; i < MF::NACC; ++i) {
                    const int grow = wrow0 + fm * MT + MF::row(i, lane);
                    const int gcol = wcol0 + fn * MT + lane % MT;
                    if (grow < a.M && gcol < a.N)
                        unsafeAtomicAdd(C + (size_t)grow * a.N + gcol, acc[fm][fn][i]);
                }
    } else {
        float* W = (float*)a.C + (size_t)blockIdx.y * a.M * a.N;
#pragma unroll
        for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < Cfg::FN; ++fn)
#pragma unroll
                for (int i = 0; i < MF::NACC; ++i) {
                    const int grow = wrow0 + fm * MT + MF::row(i, lane);
                    const int gcol = wcol0 + fn * MT + lane % MT;
                    if (grow < a.M && gcol < a.N)
                        W[(size_t)grow * a.N + gcol] = acc[fm][fn][i];
                }
    }
}

// Host-side launch of one instantiation: grid = (tiles, slices).
template <class Cfg, int EPI, bool ALIGNED>
hipError_t launch_gemm(const GemmArgs& a, int slices, hipStream_t stream)
{
    auto kern = gemm_nt_kernel<Cfg, EPI, ALIGNED>;
    static bool attr_set = false;   // dynamic LDS above 64 KiB must be opted into
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           Cfg::LDS_BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int tiles = ceil_div(a.M, Cfg::BM) * ceil_div(a.N, Cfg::BN);
    hipLaunchKernelGGL(kern, dim3(tiles, slices, 1), dim3(Cfg::NT, 1, 1), Cfg::LDS_BYTES, stream, a);
    return hipGetLastError();
}

}  // namespace gf
