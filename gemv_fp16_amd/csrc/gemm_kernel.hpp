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
//    rows of BK/8 chunks; chunk c of row r sits at slot c ^ swz(r).  The LDS
//    serves a 128-bit read 16 lanes (256 bytes, all 64 banks) at a time, and
//    the 16 lanes of an MFMA operand fetch read the same chunk of 16
//    consecutive rows; swz(r) = (r / (16 / CH)) % CH puts those 16 chunks in
//    16 different 16-byte bank slots (rows that share a 256-byte window get
//    the same key, rows in different windows get different keys).
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
    int kt_per_slice;   // K tiles per split-K slice
    int raster;         // 0: plain tile order; > 0: XCD remap + panel of this many rows
    int slices;         // split-K slices (set by launch_gemm); the grid is (tiles, slices)
};

// 16 zero bytes: the source of direct-to-LDS chunks that lie beyond K.
static __device__ __attribute__((aligned(16))) uint32_t g_zero16[4] = {0u, 0u, 0u, 0u};

// SCHED 0: every wave interleaves its loads with its MFMAs.  SCHED 1: two
// wave groups alternate memory and MFMA phases ("ping-pong"; 8 waves, 2x4
// wave grid, at least 2 stages).  SCHED 2: one wave per SIMD (4 waves) with
// the tile barrier placed before the last MFMA step of each K tile, so that
// the next tile's first fragments and the loads into the freed stage are
// issued under that step's MFMAs.  SCHED 3: SCHED 2 with 16x16x32 MFMAs.
// LA_ / LB_: operand layouts (0: A is M x K / B is N x K, K contiguous;
// 1: A is K x M / B is K x N, K the slow index).
template <int BM_, int BN_, int BK_, int STAGES_, int NT_, int SCHED_ = 0, int LA_ = 0, int LB_ = 0>
struct GemmCfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, STAGES = STAGES_, NT = NT_, SCHED = SCHED_;
    static constexpr int LA = LA_, LB = LB_;
    static constexpr int NWAVES = NT / kWave;
    // Square-ish wave grid; the longer tile side gets more waves.
    static constexpr int WM = (NWAVES == 4) ? 2 : (NWAVES == 8 ? (BM > BN ? 4 : 2) : 1);
    static constexpr int WN = NWAVES / WM;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int MT =                                // MFMA tile
        (SCHED != 3 && WTM % 32 == 0 && WTN % 32 == 0) ? 32 : 16;
    static constexpr int KS = (MT == 32) ? 16 : 32;                          // MFMA K
    static constexpr int FM = WTM / MT, FN = WTN / MT;
    static constexpr int CH = BK / 8;                        // 16-byte chunks per row
    static constexpr int ROWS_PER_SWZ = 16 / CH;             // rows sharing one swizzle key
    static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LPS = (BM + BN) * CH / NT;          // 16-byte loads per thread per stage
    static constexpr int EPAD = 8;                           // fp16 pad per epilogue row
    static constexpr int EPI_BYTES = NWAVES * WTM * (WTN + EPAD) * 2;
    static constexpr int MAIN_BYTES = STAGES * STAGE_BYTES;
    static constexpr int LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;

    // A config is legal when it maps onto wave64 MFMA tiles, splits evenly
    // over the loader, and fits one CU's 160 KiB of LDS.  A K-major operand
    // needs at least 16 chunks per k-row for its swizzle.
    static constexpr bool kValid =
        (NWAVES == 4 || NWAVES == 8) && WTM % MT == 0 && WTN % MT == 0 && WTM >= 16 &&
        WTN >= 16 && BK % KS == 0 && (CH == 4 || CH == 8) && ((BM + BN) * CH) % NT == 0 &&
        (BM * CH) % kWave == 0 && STAGES >= 1 && STAGES <= (SCHED >= 2 ? 5 : 4) &&
        LDS_BYTES <= 160 * 1024 &&
        LPS * (STAGES > 2 ? STAGES - 2 : 0) < 64 && (WTM * (WTN / 8)) % kWave == 0 &&
        (SCHED == 0 ||
         (SCHED == 1 && NWAVES == 8 && WM == 2 && STAGES >= 2 && LPS * (STAGES - 1) < 64) ||
         ((SCHED == 2 || SCHED == 3) && NWAVES == 4 && STAGES >= 2 && (BK / KS) % 2 == 0 &&
          LPS % 2 == 0 && LPS * STAGES < 64)) &&
        (LA == 0 || BM % 128 == 0) && (LB == 0 || BN % 128 == 0);
};

// ---------------------------------------------------------------------------
// Operand layouts
// ---------------------------------------------------------------------------
//
// Layout 0 (A: M x K, B: N x K; K contiguous): the LDS tile is [rows][BK];
// chunk c of row r (16 bytes = 8 fp16 along K) sits at slot c ^ swz(r) of
// its row.
// Layout 1 (A: K x M, B: K x N; M or N contiguous): the LDS tile is
// [BK][rows]; chunk c of k-row k (8 fp16 along M or N) sits at slot
// c ^ (4 * (k % 4)) of that k-row.  A fragment (8 consecutive k for one
// row) is gathered by two transposing reads, each of which hands every lane
// 4 values from 4 consecutive k-rows (see FragReader).

template <class Cfg, bool IS_A>
struct OperandGeom {
    static constexpr int L = IS_A ? Cfg::LA : Cfg::LB;
    static constexpr int ROWS = IS_A ? Cfg::BM : Cfg::BN;      // tile extent along M or N
    static constexpr int CR = ROWS / 8;                        // layout 1: chunks per k-row
};

// Diagnostic build only (build.py --variant timeline): each workgroup of a
// two-pass split-K launch or an fp16 GEMM notes the shader's real-time
// counter (100 MHz) on entry, once its first K tile has landed, when its main
// loop ends and after its stores, the shader-clock cycle counter at the first
// three of those points, and writes them with its XCC id over the first words
// of its own partial or output tile -- the results are then wrong by design.
// Compiled out of the library.
#ifdef GF_DIAG_TIMELINE
#define GF_STAMP(t) ((t) = __builtin_amdgcn_s_memrealtime())
#define GF_CYCLES(t) ((t) = __builtin_amdgcn_s_memtime())
#else
#define GF_STAMP(t) ((void)0)
#define GF_CYCLES(t) ((void)0)
#endif

__device__ __forceinline__ int swz_key(int row, int rows_per_key, int ch)
{
#ifdef GF_DIAG_NO_LDS_SWIZZLE
    // Diagnostic build only (build.py --variant noswizzle): the unswizzled
    // layout, kept so that its bank conflicts can be counted.
    (void)row; (void)rows_per_key; (void)ch;
    return 0;
#else
    return (row / rows_per_key) % ch;
#endif
}

// Where the 16-byte LDS slot s of an operand tile (0 <= s < rows * BK / 8)
// comes from: tile row (M/N index) and K offset of its 8 elements for
// layout 0, or k-row and M/N offset for layout 1.
template <class Cfg, int L, int ROWS>
__device__ __forceinline__ void slot_source(int s, int& k_in_tile, int& row_in_tile)
{
    if constexpr (L == 0) {
        const int row = s / Cfg::CH;
        row_in_tile = row;
        k_in_tile = ((s % Cfg::CH) ^ swz_key(row, Cfg::ROWS_PER_SWZ, Cfg::CH)) * 8;
    } else {
        constexpr int CR = ROWS / 8;
        const int k = s / CR;
        k_in_tile = k;
        row_in_tile = ((s % CR) ^ (4 * (k % 4))) * 8;
    }
}

// ---------------------------------------------------------------------------
// Operand staging
// ---------------------------------------------------------------------------

// Direct-to-LDS loader of one thread.  Load r (0 <= r < LPS) of a K tile
// fills LDS slot r * NT + tid; a wave instruction fills 64 consecutive slots,
// so the LDS address is wave-uniform and the swizzle is applied on the global
// side.  The A/B boundary is a multiple of 64 slots, so each wave
// instruction stays within one operand.  Each load's byte offset at k = 0 is
// computed once per tile position; the K tile's offset (k0 times the byte
// stride of one k step: 2 for layout 0, 2 * M or 2 * N for layout 1) is added
// per issue.
template <class Cfg>
struct DmaLoader {
    uint32_t voff[Cfg::LPS];   // byte offset of load r's chunk at k = 0 (rows / columns clamped)
    int tid;
    uint32_t ska, skb;         // bytes per k step in A and in B
    int klim;                  // K index where this workgroup's loads stop: K, or its split-K slice's end
    // Buffer descriptors of A and B (raw, byte-addressed): the tile's K
    // offset travels in the scalar offset, the row/chunk offset in voff.
    __amdgpu_buffer_rsrc_t ra, rb;

    __device__ __forceinline__ void init(const GemmArgs& a, int m0, int n0, int tid_, int klim_)
    {
        tid = tid_;
        klim = klim_;
        ska = Cfg::LA ? (uint32_t)a.M * 2u : 2u;
        skb = Cfg::LB ? (uint32_t)a.N * 2u : 2u;
#pragma unroll
        for (int r = 0; r < Cfg::LPS; ++r) {
            const int slot = r * Cfg::NT + tid;
            const bool is_a = slot < Cfg::BM * Cfg::CH;
            const int s = is_a ? slot : slot - Cfg::BM * Cfg::CH;
            int kk, rr;
            uint32_t off;
            if (is_a) {
                slot_source<Cfg, Cfg::LA, Cfg::BM>(s, kk, rr);
                off = Cfg::LA == 0 ? (uint32_t)(min(m0 + rr, a.M - 1) * a.K + kk)
                                   : (uint32_t)(kk * a.M + min(m0 + rr, a.M - 8));
            } else {
                slot_source<Cfg, Cfg::LB, Cfg::BN>(s, kk, rr);
                off = Cfg::LB == 0 ? (uint32_t)(min(n0 + rr, a.N - 1) * a.K + kk)
                                   : (uint32_t)(kk * a.N + min(n0 + rr, a.N - 8));
            }
            voff[r] = off * 2u;
        }
        constexpr int kRawBufferWord3 = 0x00020000;
        ra = __builtin_amdgcn_make_buffer_rsrc((void*)a.A, 0, (int)((uint32_t)a.M * (uint32_t)a.K * 2u),
                                               kRawBufferWord3);
        rb = __builtin_amdgcn_make_buffer_rsrc((void*)a.B, 0, (int)((uint32_t)a.N * (uint32_t)a.K * 2u),
                                               kRawBufferWord3);
    }

    // Whether load r of the K tile at k0 lies before klim (its chunk for
    // layout 0, its k-row for layout 1).
    __device__ __forceinline__ bool in_k(const GemmArgs& a, int k0, int r) const
    {
        const int slot = r * Cfg::NT + tid;
        const bool is_a = slot < Cfg::BM * Cfg::CH;
        const int s = is_a ? slot : slot - Cfg::BM * Cfg::CH;
        int kk, rr;
        if (is_a) slot_source<Cfg, Cfg::LA, Cfg::BM>(s, kk, rr);
        else slot_source<Cfg, Cfg::LB, Cfg::BN>(s, kk, rr);
        (void)a;
        return k0 + kk < klim;
    }

    // Kernels with a K-major operand read it with transposing LDS reads,
    // which the compiler cannot tell apart from the LDS bytes that a
    // pending direct-to-LDS load may still write: it would drain every load
    // in flight before each of them.  There the loads are issued as inline
    // assembly, invisible to that analysis; visibility is ordered by the
    // kernel's own vmcnt waits and barriers, as for every load here.  The
    // wave's LDS destination goes in through M0 (the compiler writes it);
    // an s_nop gives the one wait state an M0 write needs before an LDS DMA.
    static constexpr bool kAsmDma = Cfg::LA != 0 || Cfg::LB != 0;

    // Load r of the K tile whose first K index is k0; every chunk must lie
    // inside K.  Uniform base + 32-bit offset.
    __device__ __forceinline__ void issue(const GemmArgs& a, GF_LDS char* stage, int k0, int r,
                                          int wave) const
    {
        const int wslot = r * Cfg::NT + wave * kWave;    // wave-uniform
        const bool is_a = wslot < Cfg::BM * Cfg::CH;     // wave-uniform
        const uint32_t koff = (uint32_t)k0 * (is_a ? ska : skb);
        (void)a;
        if constexpr (kAsmDma) {
            const uint32_t lds = (uint32_t)(uintptr_t)(stage + wslot * 16);
            asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                         :: "{m0}"(lds), "v"(voff[r]), "s"(is_a ? ra : rb), "s"(koff));
        } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? ra : rb, (GF_LDS void*)(stage + wslot * 16),
                                                     16, voff[r], koff, 0, 0);
        }
    }

    // The same where the tile may run past klim: chunks at k >= klim read 16
    // zero bytes.
    __device__ __forceinline__ void issue_masked(const GemmArgs& a, GF_LDS char* stage, int k0, int r,
                                                 int wave) const
    {
        const int wslot = r * Cfg::NT + wave * kWave;
        const bool is_a = wslot < Cfg::BM * Cfg::CH;
        const char* base = (const char*)(is_a ? a.A : a.B);
        const void* src = in_k(a, k0, r)
                              ? (const void*)(base + voff[r] + (size_t)k0 * (is_a ? ska : skb))
                              : (const void*)g_zero16;
        if constexpr (kAsmDma) {
            const uint32_t lds = (uint32_t)(uintptr_t)(stage + wslot * 16);
            asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %1, off" :: "{m0}"(lds), "v"(src));
        } else {
            __builtin_amdgcn_global_load_lds(src, (GF_LDS void*)(stage + wslot * 16), 16, 0, 0);
        }
    }

    __device__ __forceinline__ void issue_all(const GemmArgs& a, GF_LDS char* stage, int k0,
                                              int wave) const
    {
#pragma unroll
        for (int r = 0; r < Cfg::LPS; ++r) issue(a, stage, k0, r, wave);
    }

    // Loads R0 .. R1-1 of the K tile at k0; where the tile runs past klim,
    // chunks at k >= klim read 16 zero bytes (so do all chunks of a tile
    // that lies wholly beyond it: a split-K slice's pipeline tail then reads
    // no operand bytes of the next slice).
    template <int R0, int R1>
    __device__ __forceinline__ void issue_range(const GemmArgs& a, GF_LDS char* stage, int k0,
                                                int wave) const
    {
        if (k0 + Cfg::BK <= klim) {
            static_for<R1 - R0>([&](auto j) { issue(a, stage, k0, R0 + decltype(j)::value, wave); });
        } else {
            static_for<R1 - R0>([&](auto j) { issue_masked(a, stage, k0, R0 + decltype(j)::value, wave); });
        }
    }

    __device__ __forceinline__ void issue_all_masked(const GemmArgs& a, GF_LDS char* stage, int k0,
                                                     int wave) const
    {
#pragma unroll
        for (int r = 0; r < Cfg::LPS; ++r) issue_masked(a, stage, k0, r, wave);
    }
};

// Masked staging through registers for operands that are not 16-byte
// aligned or whose K (layout 0) or M/N (layout 1) is not a multiple of 8:
// element loads with bounds checks, zero fill, then one 16-byte LDS write
// per chunk.
template <class Cfg>
__device__ __forceinline__ void load_tile_masked(const GemmArgs& a, GF_LDS char* stage, int m0,
                                                 int n0, int k0, int tid)
{
#pragma unroll
    for (int r = 0; r < Cfg::LPS; ++r) {
        const int slot = r * Cfg::NT + tid;
        const bool is_a = slot < Cfg::BM * Cfg::CH;
        const int s = is_a ? slot : slot - Cfg::BM * Cfg::CH;
        const int L = is_a ? Cfg::LA : Cfg::LB;
        int kk, rr;
        if (is_a) slot_source<Cfg, Cfg::LA, Cfg::BM>(s, kk, rr);
        else slot_source<Cfg, Cfg::LB, Cfg::BN>(s, kk, rr);
        const int rows = is_a ? a.M : a.N;
        const int row0 = (is_a ? m0 : n0) + rr;   // layout 0: the row; layout 1: first of 8 rows
        const uint16_t* base = is_a ? a.A : a.B;
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bool ok;
            size_t idx;
            if (L == 0) {
                const int kx = k0 + kk + e;
                ok = row0 < rows && kx < a.K;
                idx = (size_t)row0 * a.K + kx;
            } else {
                const int kx = k0 + kk;
                ok = kx < a.K && row0 + e < rows;
                idx = (size_t)kx * rows + row0 + e;
            }
            v[e] = ok ? base[idx] : (uint16_t)0;
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

typedef short short4v __attribute__((ext_vector_type(4)));

// Fragment reads of one operand.  An MFMA operand gives lane l the 8
// consecutive k values kb .. kb + 7 (kb = 8 * (l / MT) within the step) of
// tile row l % MT.
//  * Layout 0: those 8 values are one swizzled 16-byte chunk: one
//    ds_read_b128.
//  * Layout 1: they lie in 8 k-rows.  ds_read_b64_tr_b16 treats each group
//    of 16 lanes as a 16 x 4 block (lane r names 4 consecutive fp16 at its
//    address) and hands lane j the values at (4 i + j / 4, j % 4), i = 0..3.
//    Lane r therefore addresses k-row kb + 4 h + r / 4 at row offset
//    16 * ((l % MT) / 16) + 4 * (r % 4), for h = 0 and 1: lane j receives 4
//    consecutive k of row 16 * ((l % MT) / 16) + j.  The four k-rows that a
//    16-lane group reads together have distinct k % 4, so the chunk swizzle
//    spreads the 32 lanes of one LDS cycle over all 64 banks.
template <class Cfg, bool IS_A>
struct FragReader {
    typedef OperandGeom<Cfg, IS_A> G;
    static constexpr int MT = Cfg::MT, L = G::L, ROWS = G::ROWS;
    static constexpr int WT = IS_A ? Cfg::WTM : Cfg::WTN;
    static constexpr int NDS = L == 0 ? 1 : 2;   // LDS instructions per fragment
    int o;       // lane part of the byte offset within the operand tile
    int q;       // layout 0: lane's K chunk group; layout 1: lane's 16-byte column chunk
    int key;     // swizzle key of the lane's reads

    __device__ __forceinline__ void init(int w, int lane)
    {
        if constexpr (L == 0) {
            const int lrow = lane % MT;
            q = lane / MT;
            key = swz_key(lrow, Cfg::ROWS_PER_SWZ, Cfg::CH);
            o = (w * WT + lrow) * (Cfg::BK * 2);
        } else {
            const int r16 = lane % 16;
            o = (8 * (lane / MT) + r16 / 4) * (ROWS * 2) + (r16 & 1) * 8;
            q = (w * WT + 16 * ((lane % MT) / 16)) / 8 + (r16 % 4) / 2;
            key = 4 * (r16 / 4);
        }
    }

    // Fragment F (tile rows F * MT ..) of MFMA step KSTEP from operand tile T.
    template <int F, int KSTEP>
    __device__ __forceinline__ half8 read(const GF_LDS char* T) const
    {
        if constexpr (L == 0) {
            return *(const GF_LDS half8*)(T + o + F * MT * (Cfg::BK * 2) +
                                          (((KSTEP * (Cfg::KS / 8) + q) ^ key) * 16));
        } else {
            const GF_LDS char* p = T + o + (((q + F * MT / 8) ^ key) << 4);
            constexpr int k0b = KSTEP * Cfg::KS * (ROWS * 2);
            const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (GF_LDS short4v*)(p + k0b));
            const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (GF_LDS short4v*)(p + k0b + 4 * ROWS * 2));
            return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    }
};

template <class Cfg>
struct Frags {
    FragReader<Cfg, true> ra;
    FragReader<Cfg, false> rb;
    __device__ __forceinline__ void init(int wm, int wn, int lane)
    {
        ra.init(wm, lane);
        rb.init(wn, lane);
    }
    template <int KSTEP>
    __device__ __forceinline__ void load_all(const GF_LDS char* stage, half8 (&af)[Cfg::FM],
                                             half8 (&bf)[Cfg::FN]) const
    {
        static_for<Cfg::FM>([&](auto f) { af[f] = ra.template read<decltype(f)::value, KSTEP>(stage); });
        static_for<Cfg::FN>([&](auto f) {
            bf[f] = rb.template read<decltype(f)::value, KSTEP>(stage + Cfg::A_BYTES);
        });
    }
};

// sched_group_barrier instruction classes
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedDsRead = 0x100;

// All MFMA steps of one K tile, with two kinds of memory traffic woven into
// the MFMA stream instead of being issued in bursts:
//  * fragments are double-buffered in registers: the LDS reads of step ks+1
//    go out between the first MFMAs of step ks;
//  * the direct-to-LDS loads of a later K tile (when LOAD) are spread
//    one per few MFMAs over the first half of the steps.  A burst of them
//    backs up the address path and stalls the issuing wave, and with it the
//    wave's matrix core.
template <class Cfg, bool LOAD>
__device__ __forceinline__ void compute_tile(const GF_LDS char* stage, const Frags<Cfg>& fr,
                                             typename Mfma<Cfg::MT>::acc_t (&acc)[Cfg::FM][Cfg::FN],
                                             const GemmArgs& a, const DmaLoader<Cfg>& ld,
                                             GF_LDS char* lstage, int lk0, int wave)
{
    constexpr int MT = Cfg::MT;
    constexpr int KSTEPS = Cfg::BK / Cfg::KS;
    constexpr int NM = Cfg::FM * Cfg::FN;                  // MFMAs per step
    constexpr int ND = Cfg::FM + Cfg::FN;                  // fragment reads per step
    constexpr int LSTEPS = KSTEPS >= 2 ? KSTEPS / 2 : 1;   // steps that carry tile loads
    constexpr int NV = (Cfg::LPS + LSTEPS - 1) / LSTEPS;   // tile loads per such step
    constexpr int SP = NM / NV > 0 ? NM / NV : 1;          // MFMAs between two tile loads
    const GF_LDS char* Bt = stage + Cfg::A_BYTES;
    half8 af[2][Cfg::FM], bf[2][Cfg::FN];
    fr.template load_all<0>(stage, af[0], bf[0]);
    static_for<KSTEPS>([&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        constexpr int cur = ks & 1;
        constexpr int nks = ks + 1 < KSTEPS ? ks + 1 : ks;
        auto read = [&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            if constexpr (i < Cfg::FM)
                af[cur ^ 1][i] = fr.ra.template read<i, nks>(stage);
            else
                bf[cur ^ 1][i - Cfg::FM] = fr.rb.template read<i - Cfg::FM, nks>(Bt);
        };
        auto nds = [](int i) constexpr {
            return i < Cfg::FM ? FragReader<Cfg, true>::NDS : FragReader<Cfg, false>::NDS;
        };
        // Which tile load (if any) follows MFMA i of this step.
        auto load_at = [](int i) constexpr {
            return (LOAD && ks < LSTEPS && i % SP == 0 && i / SP < NV &&
                    ks * NV + i / SP < Cfg::LPS) ? ks * NV + i / SP : -1;
        };
        static_for<NM>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            constexpr int fm = i / Cfg::FN, fn = i % Cfg::FN;
            acc[fm][fn] = Mfma<MT>::run(af[cur][fm], bf[cur][fn], acc[fm][fn]);
            if constexpr (ks + 1 < KSTEPS && i < ND) read(i_c);
            if constexpr (load_at(i) >= 0)
                ld.issue(a, lstage, lk0, load_at(i), wave);
        });
        // Fragment reads that found no MFMA to follow (FM * FN < FM + FN).
        static_for<ND>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            if constexpr (ks + 1 < KSTEPS && i >= NM) read(i_c);
        });
        static_for<NM>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if constexpr (ks + 1 < KSTEPS && i < ND)
                __builtin_amdgcn_sched_group_barrier(kSchedDsRead, nds(i), 0);
            if constexpr (load_at(i) >= 0)
                __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
        });
        __builtin_amdgcn_sched_barrier(0);
    });
    // Tile loads that found no slot in the MFMA stream (only when a step has
    // more loads than MFMAs).
    if constexpr (LOAD && NV > (NM + SP - 1) / SP) {
        static_for<LSTEPS>([&](auto ks_c) {
            constexpr int ks = decltype(ks_c)::value;
            static_for<NV>([&](auto j_c) {
                constexpr int j = decltype(j_c)::value;
                if constexpr (j >= (NM + SP - 1) / SP && ks * NV + j < Cfg::LPS)
                    ld.issue(a, lstage, lk0, ks * NV + j, wave);
            });
        });
    }
}

// One MFMA step of SCHED 2/3: the FM x FN MFMAs on fragment buffer CUR,
// with the reads of step RKS's fragments from stage RS (possibly the next
// tile's) into buffer CUR ^ 1 and the direct-to-LDS loads R0 .. R1-1 of the
// tile at lk0 woven into the stream.
template <class Cfg, int CUR, int RKS, int R0, int R1>
__device__ __forceinline__ void mfma_step(typename Mfma<Cfg::MT>::acc_t (&acc)[Cfg::FM][Cfg::FN],
                                          half8 (&af)[2][Cfg::FM], half8 (&bf)[2][Cfg::FN],
                                          const Frags<Cfg>& fr, const GF_LDS char* RS,
                                          const GemmArgs& a, const DmaLoader<Cfg>& ld,
                                          GF_LDS char* lstage, int lk0, int wave)
{
    constexpr int MT = Cfg::MT;
    constexpr int NM = Cfg::FM * Cfg::FN, ND = Cfg::FM + Cfg::FN, NL = R1 - R0;
    constexpr int SP = NL > 0 ? (NM >= NL ? NM / (NL > 0 ? NL : 1) : 1) : NM + 1;  // MFMAs per load
    constexpr int NLS = NL > 0 ? (NM + SP - 1) / SP : 0;                // loads in the stream
    auto load_at = [](int i) constexpr {
        return (i % SP == 0 && i / SP < NL) ? R0 + i / SP : -1;
    };
    // Read j fetches the fragment that the next step needs j-th: the MFMAs
    // run row by row (A[fm] x B[0..FN-1]), so B0 and A0 first, then the
    // rest of B, then A1 .. A[FM-1].  Each MFMA then waits only for its own
    // operands instead of for the whole batch.
    // LDS instructions behind read j (the read that follows MFMA j).
    auto nds = [](int j) constexpr {
        return ((j == 0) || (j >= 2 && j <= Cfg::FN)) ? FragReader<Cfg, false>::NDS
                                                      : FragReader<Cfg, true>::NDS;
    };
    const GF_LDS char* RBt = RS + Cfg::A_BYTES;
    auto read = [&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        constexpr bool b = (j == 0) || (j >= 2 && j <= Cfg::FN);
        constexpr int f = (j == 0 || j == 1) ? 0 : (b ? j - 1 : j - Cfg::FN);
        if constexpr (b)
            bf[CUR ^ 1][f] = fr.rb.template read<f, RKS>(RBt);
        else
            af[CUR ^ 1][f] = fr.ra.template read<f, RKS>(RS);
    };
    static_for<NM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int fm = i / Cfg::FN, fn = i % Cfg::FN;
        acc[fm][fn] = Mfma<MT>::run(af[CUR][fm], bf[CUR][fn], acc[fm][fn]);
        if constexpr (i < ND) read(i_c);
        if constexpr (load_at(i) >= 0) ld.issue(a, lstage, lk0, load_at(i), wave);
    });
    static_for<ND>([&](auto j_c) {
        if constexpr (decltype(j_c)::value >= NM) read(j_c);
    });
    static_for<NL>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        if constexpr (j >= NLS) ld.issue(a, lstage, lk0, R0 + j, wave);
    });
    static_for<NM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int nr = i < ND ? nds(i) : 0;
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, nr, 0);
        if constexpr (load_at(i) >= 0) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    });
    __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// Ping-pong phases (SCHED 1)
// ---------------------------------------------------------------------------

// Memory phase, part 1: every fragment this wave needs for one K tile, read
// from LDS into registers (FM + FN reads per MFMA step).
template <class Cfg>
__device__ __forceinline__ void read_tile_frags(const GF_LDS char* stage, const Frags<Cfg>& fr,
                                                half8 (&af)[Cfg::BK / Cfg::KS][Cfg::FM],
                                                half8 (&bf)[Cfg::BK / Cfg::KS][Cfg::FN])
{
    static_for<Cfg::BK / Cfg::KS>([&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        fr.template load_all<ks>(stage, af[ks], bf[ks]);
    });
}

// MFMA phase: the whole K tile from registers, nothing else in the stream.
template <class Cfg>
__device__ __forceinline__ void mfma_tile(typename Mfma<Cfg::MT>::acc_t (&acc)[Cfg::FM][Cfg::FN],
                                          const half8 (&af)[Cfg::BK / Cfg::KS][Cfg::FM],
                                          const half8 (&bf)[Cfg::BK / Cfg::KS][Cfg::FN])
{
    static_for<Cfg::BK / Cfg::KS>([&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        static_for<Cfg::FM * Cfg::FN>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            constexpr int fm = i / Cfg::FN, fn = i % Cfg::FN;
            acc[fm][fn] = Mfma<Cfg::MT>::run(af[ks][fm], bf[ks][fn], acc[fm][fn]);
        });
    });
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <class Cfg, int EPI, bool ALIGNED>
__global__ __launch_bounds__(Cfg::NT) void gemm_nt_kernel(GemmArgs a)
{
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
    typedef Mfma<Cfg::MT> MF;
    typedef typename MF::acc_t acc_t;
    extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
    GF_LDS char* smem = (GF_LDS char*)smem_raw;
    [[maybe_unused]] uint64_t ts0 = 0, ts1 = 0, ts2 = 0, cy0 = 0, cy1 = 0, cy2 = 0;
    GF_STAMP(ts0);
    GF_CYCLES(cy0);

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

    // ---- which tile, and which K slice ----
    const int tiles_m = ceil_div(a.M, Cfg::BM), tiles_n = ceil_div(a.N, Cfg::BN);
    const int ntiles = tiles_m * tiles_n;
    int tm, tn, slice = 0;
    int w = blockIdx.x;
    if (a.slices > 1) {
        // Split-K: the grid (tiles, slices) enumerates (slice, tile) work
        // items slice by slice in dispatch order.  With the XCD remap each
        // XCD receives one contiguous run of items -- every tile of one K
        // slice (or of a few) -- so the A and B panels of that K range are
        // fetched into the XCD's L2 once and shared by its workgroups,
        // instead of every XCD streaming the whole K extent of a few tiles.
        w += blockIdx.y * gridDim.x;
        const int L = a.raster > 0 ? xcd_remap(w, ntiles * a.slices) : w;
        slice = L / ntiles;
        w = L - slice * ntiles;
        tm = w / tiles_n;
        tn = w % tiles_n;
    } else if (a.raster > 0) {
        grouped_tile(xcd_remap(w, ntiles), tiles_m, tiles_n, a.raster, tm, tn);
    } else {
        tm = w / tiles_n;
        tn = w % tiles_n;
    }
    const int m0 = tm * Cfg::BM, n0 = tn * Cfg::BN;

    // ---- which K tiles ----
    const int nkt_total = ceil_div(a.K, Cfg::BK);
    const int kt_begin = slice * a.kt_per_slice;
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
    auto k0_of = [&](int kt) { return (kt_begin + kt) * Cfg::BK; };
    DmaLoader<Cfg> ld;
    if constexpr (ALIGNED) ld.init(a, m0, n0, tid, min(a.K, kt_end * Cfg::BK));
    Frags<Cfg> fr;
    fr.init(wm, wn, lane);
    // Whole-tile load, used where nothing can overlap it (pipeline prologue,
    // single-stage configs, and the masked unaligned path).
    auto burst = [&](int s, int kt) {
        const int k0 = k0_of(kt);
        if constexpr (ALIGNED) {
            if (k0 + Cfg::BK <= a.K)
                ld.issue_all(a, stage_ptr(s), k0, wave);
            else
                ld.issue_all_masked(a, stage_ptr(s), k0, wave);
        } else {
            load_tile_masked<Cfg>(a, stage_ptr(s), m0, n0, k0, tid);
        }
    };

    if constexpr (Cfg::SCHED == 1 && ALIGNED) {
        // Ping-pong.  Group g = wm (waves 0-3 own tile rows [0, WTM), waves
        // 4-7 the rest); the two waves on a SIMD belong to different groups.
        // Both groups run the same loop -- M phase (read this tile's
        // fragments into registers, issue this wave's share of the loads of
        // tile t + D, D = STAGES - 1), barrier, C phase (MFMAs only), barrier
        // -- with group 1 one phase behind group 0, so that on every SIMD one
        // wave multiplies while the other moves data.  Stage (t + D) % STAGES
        // last held tile t - 1, which both groups finished reading before
        // the barrier that opens group 0's M phase of tile t.
        // Every wave waits for its own loads of tile t + 1 before the barrier
        // that ends each phase of tile t, so that tile is complete when the
        // next M phase reads it.
        constexpr int D = Cfg::STAGES - 1;
        constexpr int KST = Cfg::BK / Cfg::KS;
        const int g = wm;
        half8 af[KST][Cfg::FM], bf[KST][Cfg::FN];
        auto issue_tile = [&](int t) {
            const int k0 = k0_of(t);
            if (k0 + Cfg::BK <= a.K)
                ld.issue_all(a, stage_ptr(t % Cfg::STAGES), k0, wave);
            else
                ld.issue_all_masked(a, stage_ptr(t % Cfg::STAGES), k0, wave);
        };
        for (int t = 0; t < D; ++t)
            if (t < nk) issue_tile(t);
        wait_vmcnt<0>();
        lds_barrier();                           // tiles 0 .. D-1 resident
        if (g == 1) lds_barrier();               // group 1 starts one phase later
        // Steady state: tile t + D exists and lies inside K.  Loads of up to
        // D tiles may be pending; tile t + 1 must be done at each barrier, so
        // D - 1 younger tiles stay in flight.  The tail loop below takes the
        // last tiles (and a ragged final tile's loads) and drains everything;
        // the two loops are kept apart so that no wait sits under a branch
        // (a scalar s_waitcnt in a flattened branch would run on both sides).
        const int nfull = (nk > 0 && k0_of(nk - 1) + Cfg::BK > a.K) ? nk - 1 : nk;
        const int steady_end = max(0, nfull - D);
        int t = 0;
        for (; t < steady_end; ++t) {
            read_tile_frags<Cfg>(stage_ptr(t % Cfg::STAGES), fr, af, bf);
            ld.issue_all(a, stage_ptr((t + D) % Cfg::STAGES), k0_of(t + D), wave);
            wait_vmcnt<Cfg::LPS * (D - 1)>();
            lds_barrier();
            __builtin_amdgcn_s_setprio(1);
            mfma_tile<Cfg>(acc, af, bf);
            __builtin_amdgcn_s_setprio(0);
            wait_vmcnt<Cfg::LPS * (D - 1)>();
            lds_barrier();
        }
        for (; t < nk; ++t) {
            read_tile_frags<Cfg>(stage_ptr(t % Cfg::STAGES), fr, af, bf);
            if (t + D < nk) issue_tile(t + D);
            wait_vmcnt<0>();
            lds_barrier();
            __builtin_amdgcn_s_setprio(1);
            mfma_tile<Cfg>(acc, af, bf);
            __builtin_amdgcn_s_setprio(0);
            wait_vmcnt<0>();
            lds_barrier();
        }
        if (g == 0) lds_barrier();               // matches group 1's extra barrier
    } else if constexpr ((Cfg::SCHED == 2 || Cfg::SCHED == 3) && ALIGNED) {
        // One wave per SIMD.  Tile t sits in stage t % S.  Barrier B(t) comes
        // before the last MFMA step of tile t: by then every wave has read
        // all of tile t's fragments (the last step's were read during the
        // step before), and each wave has waited for its own loads of tile
        // t + 1, so after B(t) tile t + 1 is complete and stage t % S is free.
        // Under the last step's MFMAs each wave then reads tile t + 1's
        // first fragments and issues the first half of tile t + S's loads
        // into stage t % S; the second half follows in tile t + 1's first
        // step.  At B(t) the loads of tiles t + 2 .. t + S - 1 may still be
        // in flight: S - 2 tiles.  Loads are issued for every tile index,
        // also past the slice (masked ones read zeros), so that the count
        // of loads in flight, and with it every wait, is the same in every
        // iteration; no wait sits under a branch.
        constexpr int S = Cfg::STAGES;
        constexpr int KST = Cfg::BK / Cfg::KS;
        // Loads of tile t + S: half under the last step of tile t, half in
        // the first step of tile t + 1 (measured best among splits over one
        // to three steps).
        constexpr int H = Cfg::LPS / 2;
        auto rest_lo = [](int ks) constexpr { return ks >= 1 ? Cfg::LPS : H; };
        half8 af[2][Cfg::FM], bf[2][Cfg::FN];
        if (nk > 0) {
#pragma unroll
            for (int t = 0; t < S - 1; ++t)
                ld.template issue_range<0, Cfg::LPS>(a, stage_ptr(t), k0_of(t), wave);
        }
        wait_vmcnt<Cfg::LPS * (S - 2)>();       // tile 0 landed
        lds_barrier();
        GF_STAMP(ts1);
        GF_CYCLES(cy1);
        if (nk > 0) ld.template issue_range<0, H>(a, stage_ptr(S - 1), k0_of(S - 1), wave);
        fr.template load_all<0>(stage_ptr(0), af[0], bf[0]);
        // Steady state: tiles t + S - 1 and t + S lie wholly inside K, so
        // their loads go into the MFMA stream unmasked.
        const int nfull = (nk > 0 && k0_of(nk - 1) + Cfg::BK > a.K) ? nk - 1 : nk;
        const int steady_end = max(0, nfull - S);
        int t = 0;
        for (; t < steady_end; ++t) {
            const int s0 = t % S, s1 = (t + 1) % S, sl = (t + S - 1) % S;
            static_for<KST - 1>([&](auto ks_c) {
                constexpr int ks = decltype(ks_c)::value;
                mfma_step<Cfg, ks & 1, ks + 1, rest_lo(ks), rest_lo(ks + 1)>(
                    acc, af, bf, fr, stage_ptr(s0), a, ld, stage_ptr(sl), k0_of(t + S - 1), wave);
            });
            wait_vmcnt<Cfg::LPS * (S - 2)>();   // tile t + 1 landed
            lds_barrier();                       // B(t)
            mfma_step<Cfg, (KST - 1) & 1, 0, 0, H>(acc, af, bf, fr, stage_ptr(s1), a, ld,
                                                   stage_ptr(s0), k0_of(t + S), wave);
        }
        for (; t < nk; ++t) {
            const int s0 = t % S, s1 = (t + 1) % S, sl = (t + S - 1) % S;
            ld.template issue_range<H, Cfg::LPS>(a, stage_ptr(sl), k0_of(t + S - 1), wave);
            static_for<KST - 1>([&](auto ks_c) {
                constexpr int ks = decltype(ks_c)::value;
                mfma_step<Cfg, ks & 1, ks + 1, 0, 0>(acc, af, bf, fr, stage_ptr(s0), a, ld, nullptr,
                                                     0, wave);
            });
            wait_vmcnt<Cfg::LPS * (S - 2)>();
            lds_barrier();
            ld.template issue_range<0, H>(a, stage_ptr(s0), k0_of(t + S), wave);
            // After the last tile these reads fetch stale data that no MFMA uses.
            mfma_step<Cfg, (KST - 1) & 1, 0, 0, 0>(acc, af, bf, fr, stage_ptr(s1), a, ld, nullptr, 0,
                                                   wave);
        }
        wait_vmcnt<0>();                         // no load may land after the epilogue starts
    } else if constexpr (Cfg::STAGES == 1) {
        for (int kt = 0; kt < nk; ++kt) {
            lds_barrier();                       // everyone is done with the buffer
            burst(0, kt);
            wait_vmcnt<0>();
            lds_barrier();
            compute_tile<Cfg, false>(stage_ptr(0), fr, acc, a, ld, nullptr, 0, wave);
        }
    } else {
#pragma unroll
        for (int s = 0; s < Cfg::STAGES - 1; ++s)
            if (s < nk) burst(s, s);
        // Steady state: the tile fetched during tile kt is kt + STAGES - 1 and
        // lies wholly inside K, so its loads can be woven into the MFMA stream.
        // The last STAGES - 1 tiles (and a ragged final tile's fetch) run in a
        // separate drain loop; keeping the two loop bodies apart keeps the
        // register allocator from merging their live ranges.
        int fast_end = 0;
        if constexpr (ALIGNED) {
            const int nfull = (nk > 0 && k0_of(nk - 1) + Cfg::BK > a.K) ? nk - 1 : nk;
            fast_end = max(0, nfull - (Cfg::STAGES - 1));
        }
        int kt = 0;
        for (; kt < fast_end; ++kt) {
            wait_vmcnt<Cfg::LPS * (Cfg::STAGES - 2)>();    // tile kt landed
            lds_barrier();                       // tile kt visible; tile kt-1 consumed
            const int kn = kt + Cfg::STAGES - 1;
            compute_tile<Cfg, ALIGNED>(stage_ptr(kt % Cfg::STAGES), fr, acc, a, ld,
                                       stage_ptr(kn % Cfg::STAGES), k0_of(kn), wave);
        }
        for (; kt < nk; ++kt) {
            // Tile kt has landed once at most STAGES-2 younger tiles are pending.
            if (kt + Cfg::STAGES - 2 < nk)
                wait_vmcnt<Cfg::LPS * (Cfg::STAGES - 2)>();
            else
                wait_vmcnt<0>();
            lds_barrier();
            const int kn = kt + Cfg::STAGES - 1;
            if (kn < nk) burst(kn % Cfg::STAGES, kn);
            compute_tile<Cfg, false>(stage_ptr(kt % Cfg::STAGES), fr, acc, a, ld, nullptr, 0,
                                     wave);
        }
    }

    // ---- epilogue ----
    GF_STAMP(ts2);
    GF_CYCLES(cy2);
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
                // C is written once and not read back here: a streaming
                // store keeps it from displacing operand lines in L2.
                __builtin_nontemporal_store(v, (u32x4*)(C + (size_t)grow * a.N + gcol));
            } else {
                const uint32_t parts[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (gcol + e < a.N)
                        C[(size_t)grow * a.N + gcol + e] = (uint16_t)(parts[e / 2] >> (16 * (e % 2)));
            }
        }
#ifdef GF_DIAG_TIMELINE
        // The tile's first 32 outputs of row m0 are this wave's (wave 0's
        // sub-tile); once its stores are done the stamps overwrite them.
        __builtin_amdgcn_s_waitcnt(0);
        uint64_t ts3;
        GF_STAMP(ts3);
        if (tid == 0 && n0 + 32 <= a.N && ((size_t)m0 * a.N + n0) % 4 == 0) {
            uint64_t* t = (uint64_t*)(C + (size_t)m0 * a.N + n0);
            t[0] = ts0; t[1] = ts1; t[2] = ts2; t[3] = ts3;
            t[4] = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // XCC_ID
            t[5] = cy0; t[6] = cy1; t[7] = cy2;
        }
#endif
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
        float* W = (float*)a.C + (size_t)slice * a.M * a.N;
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
#ifdef GF_DIAG_TIMELINE
        __builtin_amdgcn_s_waitcnt(0);
        uint64_t ts3;
        GF_STAMP(ts3);
        if (tid == 0 && n0 + 16 <= a.N) {   // eight 8-byte words inside the tile's first row
            uint64_t* t = (uint64_t*)(W + (size_t)m0 * a.N + n0);
            t[0] = ts0; t[1] = ts1; t[2] = ts2; t[3] = ts3;
            t[4] = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // XCC_ID
            t[5] = cy0; t[6] = cy1; t[7] = cy2;
        }
#endif
    }
#endif
}

// Host-side launch of one instantiation: grid = (tiles, slices).
template <class Cfg, int EPI, bool ALIGNED>
hipError_t launch_gemm(const GemmArgs& args, int slices, hipStream_t stream)
{
    GemmArgs a = args;
    a.slices = slices;
    auto kern = gemm_nt_kernel<Cfg, EPI, ALIGNED>;
    static std::atomic<uint64_t> lds_opt_in{0};   // devices where the LDS size is opted into
    {
        const hipError_t e = opt_in_lds((const void*)kern, Cfg::LDS_BYTES, lds_opt_in, stream);
        if (e != hipSuccess) return e;
    }
    const int tiles = ceil_div(a.M, Cfg::BM) * ceil_div(a.N, Cfg::BN);
    hipLaunchKernelGGL(kern, dim3(tiles, slices, 1), dim3(Cfg::NT, 1, 1), Cfg::LDS_BYTES, stream, a);
    return hipGetLastError();
}

}  // namespace gf
