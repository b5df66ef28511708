// 2:4 structured-sparse fp16 GEMM for gfx950: C = decompress(A_sparse, E) . B^T
// with fp32 accumulation, plus the kernel that compresses a dense A.
//
// Format (TileLang FP16 matmul autotune benchmark page, section 6: A is
// compressed 2:4-style into A_sparse of shape (M, K/2) plus mask metadata E
// of shape (M, K/e_factor); the selection rule and the bit layout are this
// library's reading of it):
//  * K is cut into groups of 4 consecutive entries; each group keeps two.
//  * A_sparse (M x K/2 fp16, row-major): the kept values of group g at 2g and
//    2g+1, lower index first.
//  * E (M x K/16 16-bit words, row-major): group g's 4-bit field
//    i0 | i1 << 2 (i0 < i1, the kept indices) at bits 4 (g % 4) of word g / 4.
//    Read as bytes or 32-bit words the same memory is E with e_factor 8 or 32.
//  * Compression keeps the two entries of largest magnitude (fp16 bits
//    without the sign; NaN ranks above infinity), ties to the lower index.
//
// The GEMM uses gfx950's sparse MFMA v_smfmac_f32_32x32x32_f16.  Per lane it
// takes 8 kept A values (4 groups, one 4-bit index field each, fields in the
// low 16 bits of the index operand) and 16 dense B values, and multiplies a
// 32 x 32 output block over 32 logical k.  In the instruction's own k order,
// lane group g (lanes 32 g .. 32 g + 31) of A owns groups
// 4 (q / 2) + 2 g + q % 2 for fields q = 0..3, and lane group h of B holds
// k = 16 h .. 16 h + 15.  A dot product does not depend on the order of its
// k, so the kernel feeds each MFMA step s of a 64-wide K tile a permuted k
// order that makes every operand read a plain 16-byte LDS read:
//  * A lane group g reads compressed chunk w = 2 g + s of the tile (8 kept
//    values = groups 4w .. 4w+3, exactly metadata word w, so the index
//    operand is E's word as stored);
//  * B lane group h then needs, for instruction groups 4h .. 4h+3, the tile's
//    k ranges [16 s + 8 h, +8) and [32 + 16 s + 8 h, +8): two 16-byte chunks.
//
// Staging: A_sparse and B of one K tile go global -> LDS with direct-to-LDS
// 16-byte loads, one stage per tile in a ring.  The metadata of two K tiles
// (16 bytes per row) moves together into a separate three-slot ring with
// 4-byte direct-to-LDS loads, half a slot per K tile: a load instruction then
// covers 16 rows instead of 32, which halves the cache lines the address unit
// has to process for E (the loads, not the MFMAs, set the pace of this
// kernel).  The schedule is the dense GEMM's one-wave-per-SIMD form: the
// tile barrier sits before the last MFMA step, and the next tile's first
// fragments and half of a later tile's loads go under that step.  The paired
// form at the end of this file stages A_sparse two K tiles and the metadata
// eight K tiles at a time, beside two B stages.
#pragma once
#include "common.hpp"

namespace gf {

typedef _Float16 half16 __attribute__((ext_vector_type(16)));

struct SpArgs {
    const uint16_t* Asp;   // M x K/2 kept values
    const uint16_t* E;     // M x K/16 metadata words
    const uint16_t* B;     // N x K
    uint16_t* C;           // M x N
    int M, N, K;
    int raster;            // 0: plain tile order; > 0: XCD remap + panel of this many rows
};

// 16 zero bytes: the source of operand chunks that lie beyond K.
static __device__ __attribute__((aligned(16))) uint32_t g_sp_zero16[4] = {0u, 0u, 0u, 0u};

// ---------------------------------------------------------------------------
// Compression: one thread per metadata word (16 consecutive k of one row).
// ---------------------------------------------------------------------------

// Kept pair of one group: entry t is kept when fewer than two entries beat
// it, where u beats t if its magnitude is larger, or equal with u < t.
__device__ __forceinline__ uint32_t sp24_pick(uint32_t x01, uint32_t x23, uint32_t& vals)
{
    const uint32_t x[4] = {x01 & 0xffffu, x01 >> 16, x23 & 0xffffu, x23 >> 16};
    uint32_t m[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) m[t] = x[t] & 0x7fffu;
    int beaten[4] = {0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = u + 1; t < 4; ++t) {
            beaten[t] += m[u] >= m[t];   // u is the lower index: it wins ties
            beaten[u] += m[t] > m[u];
        }
    int i0 = 3, i1 = 3;
#pragma unroll
    for (int t = 3; t >= 0; --t)
        if (beaten[t] < 2) { i1 = i0; i0 = t; }
    vals = x[i0] | (x[i1] << 16);
    return (uint32_t)(i0 | (i1 << 2));
}

// A (words x 16 fp16 values, i.e. M x K flattened, K % 16 == 0) -> A_sparse
// (8 values per word) and E (one 16-bit word per word).  16-byte aligned A
// and A_sparse.
__global__ __launch_bounds__(256) void sp24_compress_kernel(const u32x4* __restrict__ A,
                                                            u32x4* __restrict__ Asp,
                                                            uint16_t* __restrict__ E, size_t words)
{
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t w = (size_t)blockIdx.x * 256 + threadIdx.x; w < words; w += stride) {
        const u32x4 lo = __builtin_nontemporal_load(A + 2 * w);
        const u32x4 hi = __builtin_nontemporal_load(A + 2 * w + 1);
        uint32_t v0, v1, v2, v3;
        uint32_t e = sp24_pick(lo.x, lo.y, v0);
        e |= sp24_pick(lo.z, lo.w, v1) << 4;
        e |= sp24_pick(hi.x, hi.y, v2) << 8;
        e |= sp24_pick(hi.z, hi.w, v3) << 12;
        const u32x4 v = {v0, v1, v2, v3};
        Asp[w] = v;
        E[w] = (uint16_t)e;
    }
}

// The same for operands without 16-byte alignment: 16-bit element accesses.
__global__ __launch_bounds__(256) void sp24_compress_kernel_u16(const uint16_t* __restrict__ A,
                                                                uint16_t* __restrict__ Asp,
                                                                uint16_t* __restrict__ E,
                                                                size_t words)
{
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t w = (size_t)blockIdx.x * 256 + threadIdx.x; w < words; w += stride) {
        uint32_t e = 0;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint16_t* x = A + 16 * w + 4 * g;
            uint32_t v;
            e |= sp24_pick(x[0] | ((uint32_t)x[1] << 16), x[2] | ((uint32_t)x[3] << 16), v) << (4 * g);
            Asp[8 * w + 2 * g] = (uint16_t)v;
            Asp[8 * w + 2 * g + 1] = (uint16_t)(v >> 16);
        }
        E[w] = (uint16_t)e;
    }
}

// ---------------------------------------------------------------------------
// Sparse GEMM configuration
// ---------------------------------------------------------------------------

// BM x BN output tile, K tiles of 64 logical k, STAGES LDS buffers, 4 waves
// in a 2 x 2 grid with (BM/2) x (BN/2) sub-tiles of 32 x 32 MFMA blocks.
template <int BM_, int BN_, int STAGES_>
struct SpCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64, STAGES = STAGES_, NT = 256;
    static constexpr int WM = 2, WN = 2;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KST = BK / 32;                    // sparse MFMA steps per K tile
    static constexpr int CHA = BK / 16, CHB = BK / 8;      // 16-byte chunks per row: A_sparse, B
    static constexpr int EDW = BK / 32;                    // metadata dwords per row per K tile
    static constexpr int A_BYTES = BM * CHA * 16, B_BYTES = BN * CHB * 16;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // Metadata ring: slot j holds K tiles 2j and 2j+1 of every tile row
    // (16 bytes per row, dword positions keyed by sp_ekey), three slots after
    // the operand stages.
    static constexpr int E_SLOT = BM * EDW * 4 * 2, E_SLOTS = 3;
    static constexpr int E_BASE = STAGES * STAGE_BYTES;
    // Loads per thread per K tile: A_sparse chunks, B chunks, E dwords (half a
    // metadata slot per K tile).
    static constexpr int LA = BM * CHA / NT, LB = BN * CHB / NT, LE = BM * EDW / NT;
    static constexpr int LAB = LA + LB, LPS = LAB + LE;
    static constexpr int EPAD = 8;                         // fp16 pad per epilogue row
    static constexpr int EPI_BYTES = 4 * WTM * (WTN + EPAD) * 2;
    static constexpr int MAIN_BYTES = STAGES * STAGE_BYTES + E_SLOTS * E_SLOT;
    static constexpr int LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
    static constexpr bool kValid =
        WTM % 32 == 0 && WTN % 32 == 0 && FM >= 1 && FN >= 1 && (BM * CHA) % NT == 0 &&
        (BN * CHB) % NT == 0 && (BM * EDW) % NT == 0 && STAGES >= 2 && STAGES <= 4 &&
        LPS * STAGES < 64 && LDS_BYTES <= 160 * 1024;
};

// Swizzle key of a tile row whose 16-byte chunks number ch per row: the 16
// lanes that the LDS serves together read one chunk index of 16 consecutive
// rows, and the key puts those reads in 16 different bank slots.
__device__ __forceinline__ int sp_key(int row, int ch) { return (row / (16 / ch)) % ch; }

// Metadata ring slot: row r's 16 bytes are dwords d = 2 h + g (K tile 2 j + h
// of the slot, lane group g's index words), stored at dword position
// d ^ sp_ekey(r).  A 4-byte LDS read is served 32 lanes at a time from 32
// banks; the 32 lanes of a lane group read 32 consecutive rows, 16 bytes
// apart, so without the key rows 8 apart share a bank (measured: 8 cycles per
// read instead of 2).  The key gives rows r, r + 8, r + 16 and r + 24
// different positions, which puts the 32 reads in 32 banks.
__device__ __forceinline__ int sp_ekey(int row) { return (row / 8) % 4; }

// ---------------------------------------------------------------------------
// Staging
// ---------------------------------------------------------------------------

// Load r of a thread fills slot (r - first load of its operand) * NT + tid
// of that operand's region; operand boundaries fall on whole loads, so every
// wave instruction stays inside one operand and its LDS address is
// wave-uniform.  The swizzle is applied on the global side.
template <class Cfg>
struct SpLoader {
    uint32_t voff[Cfg::LPS];   // byte offset of load r at k = 0 (rows clamped into range)
    int tid;
    __amdgpu_buffer_rsrc_t ra, rb, re;

    template <int R>
    static constexpr int kind() { return R < Cfg::LA ? 0 : (R < Cfg::LA + Cfg::LB ? 1 : 2); }
    template <int R>
    static constexpr int first() { return kind<R>() == 0 ? 0 : (kind<R>() == 1 ? Cfg::LA : Cfg::LA + Cfg::LB); }

    // Row within the tile and k offset (logical k of the chunk's first entry).
    template <int R>
    __device__ __forceinline__ void source(int& row, int& kk) const
    {
        const int s = (R - first<R>()) * Cfg::NT + tid;
        if constexpr (kind<R>() == 0) {
            row = s / Cfg::CHA;
            kk = ((s % Cfg::CHA) ^ sp_key(row, Cfg::CHA)) * 16;
        } else if constexpr (kind<R>() == 1) {
            row = s / Cfg::CHB;
            kk = ((s % Cfg::CHB) ^ sp_key(row, Cfg::CHB)) * 8;
        } else {
            // position s % 4 of the row's 16 metadata bytes of a two-tile slot
            // holds dword (s % 4) ^ key (the half's first row is a multiple of 32,
            // so the key of the row within the half is that within the tile)
            row = s / 4;
            kk = ((s % 4) ^ sp_ekey(row)) * 32;
        }
    }

    __device__ __forceinline__ void init(const SpArgs& a, int m0, int n0, int tid_)
    {
        tid = tid_;
        static_for<Cfg::LPS>([&](auto r_c) {
            constexpr int R = decltype(r_c)::value;
            int row, kk;
            source<R>(row, kk);
            if constexpr (kind<R>() == 0)        // A_sparse row: K/2 fp16 = K bytes
                voff[R] = (uint32_t)min(m0 + row, a.M - 1) * (uint32_t)a.K + (uint32_t)kk;
            else if constexpr (kind<R>() == 1)   // B row: 2K bytes
                voff[R] = ((uint32_t)min(n0 + row, a.N - 1) * (uint32_t)a.K + (uint32_t)kk) * 2u;
            else                                 // E row: K/8 bytes (rows past M read zeros or
                                                 // other rows' words; they feed no stored output)
                voff[R] = (uint32_t)(m0 + row) * (uint32_t)(a.K / 8) + (uint32_t)(kk / 8);
        });
        constexpr int kRawBufferWord3 = 0x00020000;
        ra = __builtin_amdgcn_make_buffer_rsrc((void*)a.Asp, 0, (int)((uint32_t)a.M * (uint32_t)a.K),
                                               kRawBufferWord3);
        rb = __builtin_amdgcn_make_buffer_rsrc((void*)a.B, 0, (int)((uint32_t)a.N * (uint32_t)a.K * 2u),
                                               kRawBufferWord3);
        re = __builtin_amdgcn_make_buffer_rsrc((void*)a.E, 0, (int)((uint32_t)a.M * (uint32_t)(a.K / 8)),
                                               kRawBufferWord3);
    }

    template <int R>
    __device__ __forceinline__ GF_LDS char* dest(GF_LDS char* stage, int wave) const
    {
        constexpr int base = kind<R>() == 0 ? 0 : Cfg::A_BYTES;
        return stage + base + ((R - first<R>()) * Cfg::NT + wave * kWave) * 16;
    }

    // Metadata half h: slot h / 2 (K tiles h - h % 2 and the next) of the
    // ring, rows [h % 2 * BM / 2, (h % 2 + 1) * BM / 2).  Its LDS base and the
    // part of the source offset common to all lanes (the slot's 16 bytes of
    // each row, plus the half's first row).  That part is added to the
    // per-lane offset, not passed as the scalar offset: the buffer's range
    // check covers the per-lane offset only, and halves past K (or rows past
    // M) reach beyond the end of E, where the check turns them into zeros.
    struct EHalf {
        GF_LDS char* lds;
        uint32_t soff;
    };
    __device__ __forceinline__ static EHalf e_half(GF_LDS char* smem, int h, int K)
    {
        const int j = h >> 1, hp = h & 1;
        EHalf e;
        e.lds = smem + Cfg::E_BASE + (j % Cfg::E_SLOTS) * Cfg::E_SLOT + hp * (Cfg::E_SLOT / 2);
        e.soff = (uint32_t)j * 16u + (uint32_t)(hp * (Cfg::BM / 2)) * (uint32_t)(K / 8);
        return e;
    }

    // Load R of the K tile at k0 (every chunk inside K), or of metadata half eh.
    template <int R>
    __device__ __forceinline__ void issue(GF_LDS char* stage, int k0, const EHalf& eh, int wave) const
    {
        if constexpr (kind<R>() == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (GF_LDS void*)dest<R>(stage, wave), 16, voff[R],
                                                     (uint32_t)k0, 0, 0);
        else if constexpr (kind<R>() == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (GF_LDS void*)dest<R>(stage, wave), 16, voff[R],
                                                     (uint32_t)k0 * 2u, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                re, (GF_LDS void*)(eh.lds + ((R - first<R>()) * Cfg::NT + wave * kWave) * 4), 4,
                voff[R] + eh.soff, 0, 0, 0);
    }

    // The same where the tile may run past K: operand chunks at k >= K read
    // 16 zero bytes.  Metadata words past K are loaded as they are (words of
    // the next row, or zeros past the end of E); whatever index they hold
    // selects zeros of both operands.
    template <int R>
    __device__ __forceinline__ void issue_masked(const SpArgs& a, GF_LDS char* stage, int k0, const EHalf& eh,
                                                 int wave) const
    {
        if constexpr (kind<R>() == 2) {
            issue<R>(stage, k0, eh, wave);
        } else {
            int row, kk;
            source<R>(row, kk);
            const char* base = kind<R>() == 0 ? (const char*)a.Asp : (const char*)a.B;
            const size_t koff = kind<R>() == 0 ? (size_t)k0 : (size_t)k0 * 2;
            const void* src = k0 + kk < a.K ? (const void*)(base + voff[R] + koff) : (const void*)g_sp_zero16;
            __builtin_amdgcn_global_load_lds(src, (GF_LDS void*)dest<R>(stage, wave), 16, 0, 0);
        }
    }

    template <int R0, int R1>
    __device__ __forceinline__ void issue_range(const SpArgs& a, GF_LDS char* stage, int k0, const EHalf& eh,
                                                int wave) const
    {
        if (k0 + Cfg::BK <= a.K) {
            static_for<R1 - R0>([&](auto j) { issue<R0 + decltype(j)::value>(stage, k0, eh, wave); });
        } else {
            static_for<R1 - R0>([&](auto j) { issue_masked<R0 + decltype(j)::value>(a, stage, k0, eh, wave); });
        }
    }

    // Metadata half h on its own.
    __device__ __forceinline__ void issue_e(GF_LDS char* smem, int h, int K, int wave) const
    {
        const EHalf eh = e_half(smem, h, K);
        static_for<Cfg::LE>([&](auto j) { issue<Cfg::LAB + decltype(j)::value>(nullptr, 0, eh, wave); });
    }
};

// Register-staged loads of one K tile for operands without the alignment the
// direct-to-LDS path needs: element loads with bounds checks, zero fill.
template <class Cfg>
__device__ __forceinline__ void sp_load_tile_masked(const SpArgs& a, GF_LDS char* stage, GF_LDS char* smem,
                                                    int m0, int n0, int t, int tid)
{
    const int k0 = t * Cfg::BK;
    // A_sparse chunks: 8 kept values = 16 logical k
    for (int s = tid; s < Cfg::BM * Cfg::CHA; s += Cfg::NT) {
        const int row = s / Cfg::CHA, kk = ((s % Cfg::CHA) ^ sp_key(row, Cfg::CHA)) * 16;
        const int gr = m0 + row;
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kc = (k0 + kk) / 2 + e;   // compressed column
            v[e] = (gr < a.M && 2 * kc < a.K) ? a.Asp[(size_t)gr * (a.K / 2) + kc] : (uint16_t)0;
        }
        u32x4 w = {v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                   v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
        *(GF_LDS u32x4*)(stage + s * 16) = w;
    }
    for (int s = tid; s < Cfg::BN * Cfg::CHB; s += Cfg::NT) {
        const int row = s / Cfg::CHB, kk = ((s % Cfg::CHB) ^ sp_key(row, Cfg::CHB)) * 8;
        const int gr = n0 + row;
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kx = k0 + kk + e;
            v[e] = (gr < a.N && kx < a.K) ? a.B[(size_t)gr * a.K + kx] : (uint16_t)0;
        }
        u32x4 w = {v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                   v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
        *(GF_LDS u32x4*)(stage + Cfg::A_BYTES + s * 16) = w;
    }
    GF_LDS char* eslot = smem + Cfg::E_BASE + ((t / 2) % Cfg::E_SLOTS) * Cfg::E_SLOT;
    for (int s = tid; s < Cfg::BM * Cfg::EDW; s += Cfg::NT) {
        const int row = s / Cfg::EDW, gr = m0 + row;
        const int w0 = (k0 + (s % Cfg::EDW) * 32) / 16;   // first metadata word
        uint32_t d = 0;
        if (gr < a.M) {
            if (w0 < a.K / 16) d = a.E[(size_t)gr * (a.K / 16) + w0];
            if (w0 + 1 < a.K / 16) d |= (uint32_t)a.E[(size_t)gr * (a.K / 16) + w0 + 1] << 16;
        }
        *(GF_LDS uint32_t*)(eslot + row * 16 + ((((t % 2) * 2 + s % Cfg::EDW) ^ sp_ekey(row)) * 4)) = d;
    }
}

// ---------------------------------------------------------------------------
// Fragments
// ---------------------------------------------------------------------------

template <class Cfg>
struct SpReader {
    int oa, ob;       // lane byte offsets of fragment 0 in the A and B regions
    int oe0, oe1;     // the same in a metadata slot, for its first and its second K tile
    int ka, kb;       // swizzle keys (the same for every fragment of the lane)
    int g;            // lane group

    __device__ __forceinline__ void init(int wm, int wn, int lane)
    {
        const int r = lane % 32;
        g = lane / 32;
        const int ra = wm * Cfg::WTM + r, rb = wn * Cfg::WTN + r;
        oa = ra * Cfg::CHA * 16;
        ka = sp_key(ra, Cfg::CHA);
        ob = Cfg::A_BYTES + rb * Cfg::CHB * 16;
        kb = sp_key(rb, Cfg::CHB);
        const int ke = sp_ekey(ra);              // rows ra + 32 F share it
        oe0 = ra * 16 + ((g ^ ke) * 4);
        oe1 = ra * 16 + (((2 + g) ^ ke) * 4);
    }
    template <int F, int S>
    __device__ __forceinline__ half8 a(const GF_LDS char* st) const
    {
        return *(const GF_LDS half8*)(st + oa + F * 32 * Cfg::CHA * 16 + (((2 * g + S) ^ ka) * 16));
    }
    template <int F, int S>
    __device__ __forceinline__ half16 b(const GF_LDS char* st) const
    {
        const GF_LDS char* p = st + ob + F * 32 * Cfg::CHB * 16;
        const half8 lo = *(const GF_LDS half8*)(p + (((2 * S + g) ^ kb) * 16));
        const half8 hi = *(const GF_LDS half8*)(p + (((2 * (Cfg::KST + S) + g) ^ kb) * 16));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }
    // Metadata words 2g (step 0, low half) and 2g + 1 (step 1, high half) of
    // K tile u: `et` is the lane's address of them for fragment 0 (e_tile).
    template <int F>
    __device__ __forceinline__ uint32_t e(const GF_LDS char* et) const
    {
        return *(const GF_LDS uint32_t*)(et + F * 32 * 16);
    }
    __device__ __forceinline__ const GF_LDS char* e_tile(const GF_LDS char* smem, int u) const
    {
        return smem + Cfg::E_BASE + ((u / 2) % Cfg::E_SLOTS) * Cfg::E_SLOT + ((u & 1) ? oe1 : oe0);
    }
};

template <class Cfg>
struct SpFrags {
    half8 a[Cfg::FM];
    half16 b[Cfg::FN];
};

__device__ __forceinline__ floatx16 sp_mfma(half8 a, half16 b, floatx16 c, uint32_t idx)
{
    return __builtin_amdgcn_smfmac_f32_32x32x32_f16(a, b, c, (int)idx, 0, 0);
}

constexpr int kSpSchedMfma = 0x008, kSpSchedVmemRead = 0x020, kSpSchedDsRead = 0x100;

// Compile-time plan of one MFMA step (see sp_step).
template <class Cfg, int RS, int R0, int R1>
struct SpStepPlan {
    static constexpr int NM = Cfg::FM * Cfg::FN, NL = R1 - R0;
    // Reads in the order the next step consumes them: its metadata first
    // (when RS == 0), then B0, A0, B1 .. B[FN-1], A1 .. A[FM-1].
    static constexpr int NE = RS == 0 ? Cfg::FM : 0;
    static constexpr int ND = NE + Cfg::FM + Cfg::FN;
    static constexpr bool is_b(int j) { return j >= NE && ((j - NE) == 0 || ((j - NE) >= 2 && (j - NE) <= Cfg::FN)); }
    static constexpr int frag(int j)
    {
        return j < NE ? j : (((j - NE) == 0 || (j - NE) == 1) ? 0 : (is_b(j) ? j - NE - 1 : j - NE - Cfg::FN));
    }
    static constexpr int nds(int j) { return is_b(j) ? 2 : 1; }   // LDS instructions behind read j
    static constexpr int RPM = (ND + NM - 1) / NM;                  // reads after each MFMA
    static constexpr int nr(int i)                                  // LDS instructions after MFMA i
    {
        int n = 0;
        for (int r = 0; r < RPM; ++r)
            if (i * RPM + r < ND) n += nds(i * RPM + r);
        return n;
    }
    static constexpr int SPL = NL > 0 ? (NM >= NL ? NM / NL : 1) : NM + 1;   // MFMAs per load
    static constexpr int NLS0 = NL > 0 ? (NM + SPL - 1) / SPL : 0;
    static constexpr int NLS = NLS0 < NL ? NLS0 : NL;                         // loads in the stream
    static constexpr int load_at(int i) { return (i % SPL == 0 && i / SPL < NL) ? R0 + i / SPL : -1; }
};

// One MFMA step: the FM x FN sparse MFMAs on fragments `cur` with index
// words `idx`, with two streams woven in: the fragment reads of step RS (from
// stage rst; with that tile's metadata from ret when RS == 0) into `nxt` /
// `enxt`, and the direct-to-LDS loads R0 .. R1-1 of the tile at lk0 into stage
// lst (metadata loads: half eh).
template <class Cfg, int RS, int R0, int R1>
__device__ __forceinline__ void sp_step(floatx16 (&acc)[Cfg::FM][Cfg::FN], const SpFrags<Cfg>& cur,
                                        const uint32_t (&idx)[Cfg::FM], SpFrags<Cfg>& nxt,
                                        uint32_t (&enxt)[Cfg::FM], const SpReader<Cfg>& rd,
                                        const GF_LDS char* rst, const GF_LDS char* ret,
                                        const SpLoader<Cfg>& ld, GF_LDS char* lst, int lk0,
                                        const typename SpLoader<Cfg>::EHalf& eh, int wave)
{
    typedef SpStepPlan<Cfg, RS, R0, R1> P;
    auto read = [&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        constexpr int f = P::frag(j);
        if constexpr (j < P::NE)
            enxt[f] = rd.template e<f>(ret);
        else if constexpr (P::is_b(j))
            nxt.b[f] = rd.template b<f, RS>(rst);
        else
            nxt.a[f] = rd.template a<f, RS>(rst);
    };
    static_for<P::NM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int fm = i / Cfg::FN, fn = i % Cfg::FN;
        acc[fm][fn] = sp_mfma(cur.a[fm], cur.b[fn], acc[fm][fn], idx[fm]);
        static_for<P::RPM>([&](auto r_c) {
            constexpr int j = i * P::RPM + decltype(r_c)::value;
            if constexpr (j < P::ND) read(std::integral_constant<int, j>{});
        });
        if constexpr (P::load_at(i) >= 0) ld.template issue<P::load_at(i)>(lst, lk0, eh, wave);
    });
    static_for<P::NL>([&](auto j_c) {
        constexpr int j = decltype(j_c)::value;
        if constexpr (j >= P::NLS) ld.template issue<R0 + j>(lst, lk0, eh, wave);
    });
    static_for<P::NM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        __builtin_amdgcn_sched_group_barrier(kSpSchedMfma, 1, 0);
        if constexpr (P::nr(i) > 0) __builtin_amdgcn_sched_group_barrier(kSpSchedDsRead, P::nr(i), 0);
        if constexpr (P::load_at(i) >= 0) __builtin_amdgcn_sched_group_barrier(kSpSchedVmemRead, 1, 0);
    });
    __builtin_amdgcn_sched_barrier(0);
}

// fp16 C of one wave's (WTM x WTN) block through a per-wave LDS transpose
// and 16-byte streaming stores (element stores on ragged or unaligned
// edges).  Waits at a workgroup barrier first: the LDS must be free.
template <class Cfg>
__device__ __forceinline__ void sp_store_c(const floatx16 (&acc)[Cfg::FM][Cfg::FN], const SpArgs& a,
                                           GF_LDS char* smem, int wrow0, int wcol0, int wave, int lane,
                                           bool aligned)
{
    uint16_t* C = a.C;
    lds_barrier();                                // operand buffers are free now
    constexpr int LDW = Cfg::WTN + Cfg::EPAD;     // fp16 per LDS row
    GF_LDS uint16_t* reg = (GF_LDS uint16_t*)(smem + wave * (Cfg::WTM * LDW * 2));
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                // 32 x 32 block: accumulator i of lane l is row 8 (i/4) + 4 (l/32) + i%4, column l%32
                const int r = fm * 32 + 8 * (i / 4) + 4 * (lane / 32) + (i % 4);
                const int c = fn * 32 + lane % 32;
                reg[r * LDW + c] = f32_to_f16_bits(acc[fm][fn][i]);
            }
    asm volatile("" ::: "memory");
    wait_lgkmcnt0();
    constexpr int CPR = Cfg::WTN / 8;             // 16-byte chunks per sub-tile row
    constexpr int ITERS = Cfg::WTM * CPR / kWave;
    const bool vec_ok = aligned && (a.N % 8 == 0) && (((uintptr_t)C & 15) == 0);
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int q = it * kWave + lane;
        const int r = q / CPR, cc = q % CPR;
        const u32x4 v = *(const GF_LDS u32x4*)(reg + r * LDW + cc * 8);
        const int grow = wrow0 + r, gcol = wcol0 + cc * 8;
        if (grow >= a.M) continue;
        if (vec_ok && gcol + 8 <= a.N) {
            __builtin_nontemporal_store(v, (u32x4*)(C + (size_t)grow * a.N + gcol));
        } else {
            const uint32_t parts[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2)
                if (gcol + e2 < a.N)
                    C[(size_t)grow * a.N + gcol + e2] = (uint16_t)(parts[e2 / 2] >> (16 * (e2 % 2)));
        }
    }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

// ALIGNED: A_sparse and B 16-byte aligned, E 4-byte aligned, K % 32 == 0 (so
// every row of E starts on a 4-byte boundary).  Otherwise the operands are
// staged through registers, one K tile at a time.
template <class Cfg, bool ALIGNED>
__global__ __launch_bounds__(256) void sp_gemm_kernel(SpArgs a)
{
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
    extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
    GF_LDS char* smem = (GF_LDS char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

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
    const int nk = ceil_div(a.K, Cfg::BK);

    floatx16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[fm][fn][i] = 0.0f;

    auto stage_ptr = [&](int s) { return smem + s * Cfg::STAGE_BYTES; };
    SpReader<Cfg> rd;
    rd.init(wm, wn, lane);
    SpFrags<Cfg> f0, f1;
    uint32_t e[Cfg::FM], lo[Cfg::FM], hi[Cfg::FM];

    if constexpr (ALIGNED) {
        // Tile t sits in stage t % S.  Barrier B(t) comes before the last MFMA
        // step of tile t: by then every wave has read all of tile t's
        // fragments and waited for its own loads of tile t + 1, so after B(t)
        // tile t + 1 is complete and stage t % S is free.  Under the last step
        // each wave reads tile t + 1's first fragments and metadata and issues
        // the first half of tile t + S's loads into stage t % S; the second
        // half goes under tile t + 1's first step.  Loads are issued for every
        // tile index, also past K (masked ones read zeros), so the count in
        // flight is the same in every iteration.
        // Metadata moves in halves of a two-tile ring slot: iteration t issues
        // half t + 4 (with the second half of the tile loads, so it has landed
        // by B(t + 1)); slot (t + 4) / 2 last held K tiles t - 2 and t - 1 (or
        // t - 3 and t - 2), whose metadata every wave read before B(t - 1).
        // The prologue loads halves 0 .. 3.  Every vmcnt wait below counts only
        // the operand loads of the tiles behind the one it waits for and so
        // may wait for a little more than needed, never less.
        constexpr int S = Cfg::STAGES, H = Cfg::LPS / 2;
        static_assert(H <= Cfg::LAB, "metadata loads must fall in the second half of a tile's loads");
        typedef typename SpLoader<Cfg>::EHalf EHalf;
        SpLoader<Cfg> ld;
        ld.init(a, m0, n0, tid);
        const EHalf no_e = {nullptr, 0u};
        if (nk > 0) {
            ld.issue_e(smem, 0, a.K, wave);
            ld.issue_e(smem, 1, a.K, wave);
#pragma unroll
            for (int t = 0; t < S - 1; ++t) {
                if (t == S - 2) {
                    ld.issue_e(smem, 2, a.K, wave);
                    ld.issue_e(smem, 3, a.K, wave);
                }
                ld.template issue_range<0, Cfg::LAB>(a, stage_ptr(t), t * Cfg::BK, no_e, wave);
            }
        }
        wait_vmcnt<Cfg::LAB * (S - 2)>();        // tile 0 and metadata halves 0, 1 landed
        lds_barrier();
        if (nk > 0) ld.template issue_range<0, H>(a, stage_ptr(S - 1), (S - 1) * Cfg::BK, no_e, wave);
        {
            const GF_LDS char* et = rd.e_tile(smem, 0);
            static_for<Cfg::FM>([&](auto f) { e[f] = rd.template e<decltype(f)::value>(et); });
        }
        static_for<Cfg::FM>([&](auto f) { f0.a[f] = rd.template a<decltype(f)::value, 0>(stage_ptr(0)); });
        static_for<Cfg::FN>([&](auto f) { f0.b[f] = rd.template b<decltype(f)::value, 0>(stage_ptr(0)); });
        // Steady state: tiles t + S - 1 and t + S lie wholly inside K.
        const int nfull = (nk > 0 && (nk - 1) * Cfg::BK + Cfg::BK > a.K) ? nk - 1 : nk;
        const int steady_end = max(0, nfull - S);
        int t = 0;
        for (; t < steady_end; ++t) {
            const int s0 = t % S, s1 = (t + 1) % S, sl = (t + S - 1) % S;
            const EHalf eh = SpLoader<Cfg>::e_half(smem, t + 4, a.K);
#pragma unroll
            for (int f = 0; f < Cfg::FM; ++f) { lo[f] = e[f] & 0xffffu; hi[f] = e[f] >> 16; }
            sp_step<Cfg, 1, H, Cfg::LPS>(acc, f0, lo, f1, e, rd, stage_ptr(s0), nullptr, ld, stage_ptr(sl),
                                         (t + S - 1) * Cfg::BK, eh, wave);
            wait_vmcnt<Cfg::LPS * (S - 2)>();    // tile t + 1 landed
            lds_barrier();                        // B(t)
            sp_step<Cfg, 0, 0, H>(acc, f1, hi, f0, e, rd, stage_ptr(s1), rd.e_tile(smem, t + 1), ld,
                                  stage_ptr(s0), (t + S) * Cfg::BK, no_e, wave);
        }
        for (; t < nk; ++t) {
            const int s0 = t % S, s1 = (t + 1) % S, sl = (t + S - 1) % S;
            ld.template issue_range<H, Cfg::LPS>(a, stage_ptr(sl), (t + S - 1) * Cfg::BK,
                                                 SpLoader<Cfg>::e_half(smem, t + 4, a.K), wave);
#pragma unroll
            for (int f = 0; f < Cfg::FM; ++f) { lo[f] = e[f] & 0xffffu; hi[f] = e[f] >> 16; }
            sp_step<Cfg, 1, 0, 0>(acc, f0, lo, f1, e, rd, stage_ptr(s0), nullptr, ld, nullptr, 0, no_e, wave);
            wait_vmcnt<Cfg::LPS * (S - 2)>();
            lds_barrier();
            ld.template issue_range<0, H>(a, stage_ptr(s0), (t + S) * Cfg::BK, no_e, wave);
            // After the last tile these reads fetch stale data that no MFMA uses.
            sp_step<Cfg, 0, 0, 0>(acc, f1, hi, f0, e, rd, stage_ptr(s1), rd.e_tile(smem, t + 1), ld,
                                  nullptr, 0, no_e, wave);
        }
        wait_vmcnt<0>();                          // no load may land after the epilogue starts
    } else {
        for (int t = 0; t < nk; ++t) {
            lds_barrier();                        // everyone is done with the buffer
            sp_load_tile_masked<Cfg>(a, stage_ptr(0), smem, m0, n0, t, tid);
            lds_barrier();
            const GF_LDS char* st = stage_ptr(0);
            const GF_LDS char* et = rd.e_tile(smem, t);
            static_for<Cfg::FM>([&](auto f) { e[f] = rd.template e<decltype(f)::value>(et); });
            static_for<Cfg::FM>([&](auto f) { f0.a[f] = rd.template a<decltype(f)::value, 0>(st); });
            static_for<Cfg::FN>([&](auto f) { f0.b[f] = rd.template b<decltype(f)::value, 0>(st); });
            static_for<Cfg::FM>([&](auto f) { f1.a[f] = rd.template a<decltype(f)::value, 1>(st); });
            static_for<Cfg::FN>([&](auto f) { f1.b[f] = rd.template b<decltype(f)::value, 1>(st); });
#pragma unroll
            for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < Cfg::FN; ++fn) {
                    acc[fm][fn] = sp_mfma(f0.a[fm], f0.b[fn], acc[fm][fn], e[fm] & 0xffffu);
                    acc[fm][fn] = sp_mfma(f1.a[fm], f1.b[fn], acc[fm][fn], e[fm] >> 16);
                }
        }
    }

    sp_store_c<Cfg>(acc, a, smem, m0 + wm * Cfg::WTM, n0 + wn * Cfg::WTN, wave, lane, ALIGNED);
#endif
}

template <class Cfg, bool ALIGNED>
hipError_t launch_sp_gemm(const SpArgs& a, hipStream_t stream)
{
    auto kern = sp_gemm_kernel<Cfg, ALIGNED>;
    static std::atomic<uint64_t> lds_opt_in{0};   // devices where the LDS size is opted into
    {
        const hipError_t err = opt_in_lds((const void*)kern, Cfg::LDS_BYTES, lds_opt_in, stream);
        if (err != hipSuccess) return err;
    }
    const int tiles = ceil_div(a.M, Cfg::BM) * ceil_div(a.N, Cfg::BN);
    hipLaunchKernelGGL(kern, dim3(tiles, 1, 1), dim3(Cfg::NT, 1, 1), Cfg::LDS_BYTES, stream, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Paired form
// ---------------------------------------------------------------------------
//
// The same product with fewer cache lines per loaded byte: the address unit
// handles a load instruction at a cost that grows with the number of cache
// lines it touches.  Here:
//  * A_sparse moves two K tiles at a time (128 bytes per row: one whole
//    cache line per row, 8 rows per instruction, instead of half a line of
//    16 rows) into a two-slot ring of K-tile pairs, half the pair's rows
//    under each of two consecutive K tiles;
//  * the metadata of eight K tiles (64 bytes per row) moves together into a
//    two-slot ring, an eighth of the rows under each K tile, with 4-byte
//    direct-to-LDS loads that cover 4 rows per instruction instead of 16;
//  * B keeps one LDS stage per K tile, two stages.
// Per 256 x 256 x 64 tile the loads touch 416 cache lines instead of 640.
// With two B stages every wait is for all loads in flight.  The trade: the
// smaller tiles gain from the lighter address work, while at 256 x 256 the
// shallower B pipeline costs about what it saves.
//
// Metadata slot layout: row r's 16 dwords (dword 2 w + g = words 4 w + 2 g
// and 4 w + 2 g + 1, i.e. lane group g's index words of K tile w of the
// slot) sit at dword position d ^ key(r), key(r) = (r / 2) mod (BM / 16).
// A 4-byte LDS read is served 32 lanes (one lane group, 32 consecutive rows
// 64 bytes apart) at a time from 32 banks, so rows of equal parity share a
// bank unless their positions differ: with BM = 256 the key gives the 16 rows
// of each parity 16 different positions and the read has no conflict; with
// BM = 128 the key repeats every 16 rows (the loads fill the slot in
// 16-row pieces), leaving rows r and r + 16 in one bank.

template <int BM_, int BN_, int HB_>
struct SpPairCfg {
    static constexpr int BM = BM_, BN = BN_, BK = 64, NT = 256;
    static constexpr int WM = 2, WN = 2;
    static constexpr int WTM = BM / WM, WTN = BN / WN;
    static constexpr int FM = WTM / 32, FN = WTN / 32;
    static constexpr int KST = BK / 32;                    // sparse MFMA steps per K tile
    static constexpr int CH = 8;                           // 16-byte chunks per row: A pair slot, B stage
    static constexpr int A_SLOT = BM * CH * 16, B_STAGE = BN * CH * 16;
    static constexpr int E_ROW = 64;                       // metadata bytes per row and slot (8 K tiles)
    static constexpr int E_SLOT = BM * E_ROW, E_PIECE_ROWS = BM / 8;
    static constexpr int A_BASE = 0, B_BASE = 2 * A_SLOT, E_BASE = B_BASE + 2 * B_STAGE;
    // Loads per thread per K tile: half an A pair slot, a B stage, an eighth
    // of a metadata slot.  B tile u's first HB loads go under the last MFMA
    // step of tile u - 2 (with that step's A and metadata loads), the rest
    // under the first step of tile u - 1.
    static constexpr int LA = BM * CH / 2 / NT, LB = BN * CH / NT, LE = E_PIECE_ROWS * (E_ROW / 4) / NT;
    static constexpr int HB = HB_;
    static constexpr int EPAD = 8;                         // fp16 pad per epilogue row
    static constexpr int EPI_BYTES = 4 * WTM * (WTN + EPAD) * 2;
    static constexpr int MAIN_BYTES = E_BASE + 2 * E_SLOT;
    static constexpr int LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
    static constexpr bool kValid =
        WTM % 32 == 0 && WTN % 32 == 0 && FM >= 1 && FN >= 1 && LA * NT * 2 == BM * CH &&
        LB * NT == BN * CH && LE >= 1 && LE * NT == E_PIECE_ROWS * (E_ROW / 4) && 0 <= HB && HB <= LB &&
        8 * LE + 2 * LA + LB < 64 && LDS_BYTES <= 160 * 1024;
};

template <class Cfg>
__device__ __forceinline__ int spp_ekey(int row)
{
    return (row / 2) % (Cfg::E_PIECE_ROWS / 2);
}

// Direct-to-LDS loader of the paired form.  All source offsets go in the
// per-lane offset, where the buffer's range check sees them.
template <class Cfg>
struct SppLoader {
    uint32_t va[2][Cfg::LA];   // A_sparse: load r of pair half h at k = 0 (rows clamped into range)
    uint32_t vb[Cfg::LB];      // B: load r at k = 0 (rows clamped)
    uint32_t ve[Cfg::LE];      // E: load r of eighth 0 of slot 0 (rows past M: range-checked or
                               // other rows' words; they feed no stored output)
    int tid;
    __amdgpu_buffer_rsrc_t ra, rb, re;

    // Slot s of a 128-byte-row region (A pair slot or B stage): row and the
    // 16-byte chunk of the source row that it holds.
    __device__ __forceinline__ static void chunk_source(int s, int& row, int& c)
    {
        row = s / Cfg::CH;
        c = (s % Cfg::CH) ^ sp_key(row, Cfg::CH);
    }

    __device__ __forceinline__ void init(const SpArgs& a, int m0, int n0, int tid_)
    {
        tid = tid_;
        static_for<2>([&](auto h_c) {
            constexpr int H = decltype(h_c)::value;
            static_for<Cfg::LA>([&](auto r_c) {
                int row, c;
                chunk_source(H * Cfg::BM * Cfg::CH / 2 + decltype(r_c)::value * Cfg::NT + tid, row, c);
                va[H][decltype(r_c)::value] = (uint32_t)min(m0 + row, a.M - 1) * (uint32_t)a.K + 16u * c;
            });
        });
        static_for<Cfg::LB>([&](auto r_c) {
            int row, c;
            chunk_source(decltype(r_c)::value * Cfg::NT + tid, row, c);
            vb[decltype(r_c)::value] = ((uint32_t)min(n0 + row, a.N - 1) * (uint32_t)a.K + 8u * c) * 2u;
        });
        static_for<Cfg::LE>([&](auto r_c) {
            const int s = decltype(r_c)::value * Cfg::NT + tid;
            const int row = s / 16, d = (s % 16) ^ spp_ekey<Cfg>(row);
            ve[decltype(r_c)::value] = (uint32_t)(m0 + row) * (uint32_t)(a.K / 8) + 4u * d;
        });
        constexpr int kRawBufferWord3 = 0x00020000;
        ra = __builtin_amdgcn_make_buffer_rsrc((void*)a.Asp, 0, (int)((uint32_t)a.M * (uint32_t)a.K),
                                               kRawBufferWord3);
        rb = __builtin_amdgcn_make_buffer_rsrc((void*)a.B, 0, (int)((uint32_t)a.N * (uint32_t)a.K * 2u),
                                               kRawBufferWord3);
        re = __builtin_amdgcn_make_buffer_rsrc((void*)a.E, 0, (int)((uint32_t)a.M * (uint32_t)(a.K / 8)),
                                               kRawBufferWord3);
    }

    // Load R of half H of A pair j (K tiles 2j, 2j+1) into pair slot j % 2.
    // MASKED: chunks at k >= K read 16 zero bytes.
    template <int H, int R, bool MASKED>
    __device__ __forceinline__ void issue_a(const SpArgs& a, GF_LDS char* smem, int j, int wave) const
    {
        GF_LDS char* dst = smem + Cfg::A_BASE + (j & 1) * Cfg::A_SLOT +
                           (H * Cfg::BM * Cfg::CH / 2 + R * Cfg::NT + wave * kWave) * 16;
        const uint32_t off = va[H][R] + (uint32_t)j * 128u;
        if constexpr (!MASKED) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (GF_LDS void*)dst, 16, off, 0, 0, 0);
        } else {
            int row, c;
            chunk_source(H * Cfg::BM * Cfg::CH / 2 + R * Cfg::NT + tid, row, c);
            const void* src = j * 128 + 16 * c < a.K ? (const void*)((const char*)a.Asp + off)
                                                     : (const void*)g_sp_zero16;
            __builtin_amdgcn_global_load_lds(src, (GF_LDS void*)dst, 16, 0, 0);
        }
    }

    // Load R of the B tile at k0 into stage st.
    template <int R, bool MASKED>
    __device__ __forceinline__ void issue_b(const SpArgs& a, GF_LDS char* smem, int st, int k0, int wave) const
    {
        GF_LDS char* dst = smem + Cfg::B_BASE + st * Cfg::B_STAGE + (R * Cfg::NT + wave * kWave) * 16;
        if constexpr (!MASKED) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (GF_LDS void*)dst, 16, vb[R], (uint32_t)k0 * 2u, 0, 0);
        } else {
            int row, c;
            chunk_source(R * Cfg::NT + tid, row, c);
            const void* src = k0 + 8 * c < a.K ? (const void*)((const char*)a.B + vb[R] + (size_t)k0 * 2)
                                               : (const void*)g_sp_zero16;
            __builtin_amdgcn_global_load_lds(src, (GF_LDS void*)dst, 16, 0, 0);
        }
    }

    // Load R of eighth p of metadata slot j (K tiles 8j .. 8j+7); `eoff` is
    // the eighth's and slot's part of the source offset (espan()).
    template <int R>
    __device__ __forceinline__ void issue_e(GF_LDS char* smem, int p, int j, uint32_t eoff, int wave) const
    {
        GF_LDS char* dst = smem + Cfg::E_BASE + (j & 1) * Cfg::E_SLOT +
                           (p * Cfg::E_PIECE_ROWS * 16 + R * Cfg::NT + wave * kWave) * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (GF_LDS void*)dst, 4, ve[R] + eoff, 0, 0, 0);
    }
    __device__ __forceinline__ static uint32_t espan(int p, int j, int K)
    {
        return (uint32_t)(p * Cfg::E_PIECE_ROWS) * (uint32_t)(K / 8) + (uint32_t)j * 64u;
    }

    template <int H, bool MASKED>
    __device__ __forceinline__ void issue_a_half(const SpArgs& a, GF_LDS char* smem, int j, int wave) const
    {
        static_for<Cfg::LA>([&](auto r) { issue_a<H, decltype(r)::value, MASKED>(a, smem, j, wave); });
    }
    template <int R0, int R1, bool MASKED>
    __device__ __forceinline__ void issue_b_range(const SpArgs& a, GF_LDS char* smem, int st, int k0, int wave) const
    {
        static_for<R1 - R0>([&](auto r) { issue_b<R0 + decltype(r)::value, MASKED>(a, smem, st, k0, wave); });
    }
    __device__ __forceinline__ void issue_e_piece(GF_LDS char* smem, int p, int j, int K, int wave) const
    {
        const uint32_t eoff = espan(p, j, K);
        static_for<Cfg::LE>([&](auto r) { issue_e<decltype(r)::value>(smem, p, j, eoff, wave); });
    }
};

template <class Cfg>
struct SppReader {
    int oa, ob, oe;   // lane byte offsets of fragment 0: in an A pair slot, a B stage, a metadata slot
    int qa, kb;       // A: the lane's chunk bits (2 g) ^ key; B: swizzle key
    int g, ke;        // lane group; metadata key

    __device__ __forceinline__ void init(int wm, int wn, int lane)
    {
        const int r = lane % 32;
        g = lane / 32;
        const int ra = wm * Cfg::WTM + r, rb = wn * Cfg::WTN + r;
        oa = ra * Cfg::CH * 16;
        qa = (2 * g) ^ sp_key(ra, Cfg::CH);
        ob = rb * Cfg::CH * 16;
        kb = sp_key(rb, Cfg::CH);
        oe = ra * Cfg::E_ROW;
        ke = spp_ekey<Cfg>(ra);
    }
    // Step S of K tile u (H = u % 2) from u's pair slot: compressed chunk
    // 4 H + 2 g + S of the pair's row (the bits do not overlap, so the sum is
    // an OR and commutes with the swizzle XOR).
    template <int F, int H, int S>
    __device__ __forceinline__ half8 a(const GF_LDS char* slot) const
    {
        return *(const GF_LDS half8*)(slot + oa + F * 32 * Cfg::CH * 16 + ((qa ^ (4 * H + S)) * 16));
    }
    template <int F, int S>
    __device__ __forceinline__ half16 b(const GF_LDS char* stage) const
    {
        const GF_LDS char* p = stage + ob + F * 32 * Cfg::CH * 16;
        const half8 lo = *(const GF_LDS half8*)(p + (((2 * S + g) ^ kb) * 16));
        const half8 hi = *(const GF_LDS half8*)(p + (((2 * (Cfg::KST + S) + g) ^ kb) * 16));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
    }
    // Lane offset of K tile w's dword (w = u % 8) in a metadata slot.
    __device__ __forceinline__ int eo(int w) const { return oe + (((2 * w + g) ^ ke) * 4); }
    template <int F>
    __device__ __forceinline__ uint32_t e(const GF_LDS char* slot, int eow) const
    {
        return *(const GF_LDS uint32_t*)(slot + eow + F * 32 * Cfg::E_ROW);
    }
};

// One MFMA step of the paired form: the FM x FN sparse MFMAs on `cur` with
// index words `idx`, with read(j) (read j of the next step's fragments, in
// SpStepPlan's order) and load(l) (l < NL) woven into the stream.
template <class Cfg, int RS, int NL, class Read, class Load>
__device__ __forceinline__ void spp_step(floatx16 (&acc)[Cfg::FM][Cfg::FN], const SpFrags<Cfg>& cur,
                                         const uint32_t (&idx)[Cfg::FM], Read&& read, Load&& load)
{
    typedef SpStepPlan<Cfg, RS, 0, NL> P;
    static_for<P::NM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        constexpr int fm = i / Cfg::FN, fn = i % Cfg::FN;
        acc[fm][fn] = sp_mfma(cur.a[fm], cur.b[fn], acc[fm][fn], idx[fm]);
        static_for<P::RPM>([&](auto r_c) {
            constexpr int j = i * P::RPM + decltype(r_c)::value;
            if constexpr (j < P::ND) read(std::integral_constant<int, j>{});
        });
        if constexpr (P::load_at(i) >= 0) load(std::integral_constant<int, P::load_at(i)>{});
    });
    static_for<NL>([&](auto j_c) {
        if constexpr (decltype(j_c)::value >= P::NLS) load(j_c);
    });
    static_for<P::NM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        __builtin_amdgcn_sched_group_barrier(kSpSchedMfma, 1, 0);
        if constexpr (P::nr(i) > 0) __builtin_amdgcn_sched_group_barrier(kSpSchedDsRead, P::nr(i), 0);
        if constexpr (P::load_at(i) >= 0) __builtin_amdgcn_sched_group_barrier(kSpSchedVmemRead, 1, 0);
    });
    __builtin_amdgcn_sched_barrier(0);
}

// The paired-form kernel.  Needs A_sparse and B 16-byte aligned, E 4-byte
// aligned and K % 32 == 0.
//
// Schedule (t = K tile; B(t) = the barrier before tile t's last MFMA step,
// preceded by a wait for every load in flight):
//  * step 0 of tile t: MFMAs of step 0; reads of tile t's step-1 fragments;
//    loads HB .. LB-1 of B tile t+1 (stage (t+1) % 2).
//  * B(t): tile t+1's B is complete; every wave has read all of tile t.
//  * step 1 of tile t: MFMAs of step 1; reads of tile t+1's metadata and
//    step-0 fragments; loads 0 .. HB-1 of B tile t+2 into stage t % 2, half
//    (t+1) % 2 of A pair (t+3)/2, and eighth (t+1) % 8 of metadata slot
//    (t+9)/8.
// A pair j (tiles 2j, 2j+1) is loaded under tiles 2j-3 and 2j-2, after
// B(2j-3) ended all reads of pair j-2 (tiles 2j-4, 2j-3) in the same slot,
// and has landed by B(2j-2), before tile 2j-1's last step reads tile 2j.
// Metadata slot j (tiles 8j .. 8j+7) is loaded under tiles 8j-9 .. 8j-2,
// after B(8j-9) ended the reads of slot j-2 (tile 8j-9's metadata is read
// under tile 8j-10), and has landed by B(8j-1), before tile 8j-1's last step
// reads tile 8j's metadata.  The prologue issues what tiles -1 and earlier
// would have.  Tiles past K are loaded as zeros (metadata past K: other
// rows' words or range-checked zeros, which select zeros).
template <class Cfg>
__global__ __launch_bounds__(256) void spp_gemm_kernel(SpArgs a)
{
#if defined(__HIP_DEVICE_COMPILE__)
    extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
    GF_LDS char* smem = (GF_LDS char*)smem_raw;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;

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
    const int nk = ceil_div(a.K, Cfg::BK);

    floatx16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
    for (int fm = 0; fm < Cfg::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < Cfg::FN; ++fn)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[fm][fn][i] = 0.0f;

    SppLoader<Cfg> ld;
    ld.init(a, m0, n0, tid);
    SppReader<Cfg> rd;
    rd.init(wm, wn, lane);
    auto a_slot = [&](int u) { return smem + Cfg::A_BASE + ((u >> 1) & 1) * Cfg::A_SLOT; };
    auto b_stage = [&](int st) { return smem + Cfg::B_BASE + st * Cfg::B_STAGE; };
    auto e_slot = [&](int u) { return smem + Cfg::E_BASE + ((u >> 3) & 1) * Cfg::E_SLOT; };
    SpFrags<Cfg> f0, f1;
    uint32_t e[Cfg::FM], lo[Cfg::FM], hi[Cfg::FM];

    if (nk > 0) {
#pragma unroll
        for (int p = 0; p < 8; ++p) ld.issue_e_piece(smem, p, 0, a.K, wave);
        ld.template issue_a_half<0, true>(a, smem, 0, wave);
        ld.template issue_a_half<1, true>(a, smem, 0, wave);
        ld.template issue_b_range<0, Cfg::LB, true>(a, smem, 0, 0, wave);
    }
    wait_vmcnt<0>();
    lds_barrier();
    if (nk > 0) {
        ld.template issue_b_range<0, Cfg::HB, true>(a, smem, 1, Cfg::BK, wave);
        ld.template issue_a_half<0, true>(a, smem, 1, wave);
        ld.issue_e_piece(smem, 0, 1, a.K, wave);
    }
    {
        const int eo0 = rd.eo(0);
        static_for<Cfg::FM>([&](auto f) { e[f] = rd.template e<decltype(f)::value>(e_slot(0), eo0); });
        static_for<Cfg::FM>([&](auto f) { f0.a[f] = rd.template a<decltype(f)::value, 0, 0>(a_slot(0)); });
        static_for<Cfg::FN>([&](auto f) { f0.b[f] = rd.template b<decltype(f)::value, 0>(b_stage(0)); });
    }

    // Tile t, H = t % 2 (compile-time: the loop runs tile pairs).  MASKED
    // selects the load forms that turn chunks past K into zeros.
    auto tile = [&](auto h_c, auto masked_c, int t) {
        constexpr int H = decltype(h_c)::value;
        constexpr bool MASKED = decltype(masked_c)::value;
        typedef SpStepPlan<Cfg, 1, 0, 0> P1;
        typedef SpStepPlan<Cfg, 0, 0, 0> P0;
#pragma unroll
        for (int f = 0; f < Cfg::FM; ++f) { lo[f] = e[f] & 0xffffu; hi[f] = e[f] >> 16; }
        const GF_LDS char* as0 = a_slot(t);
        const int k1 = (t + 1) * Cfg::BK;
        spp_step<Cfg, 1, Cfg::LB - Cfg::HB>(
            acc, f0, lo,
            [&](auto j_c) {
                constexpr int j = decltype(j_c)::value, f = P1::frag(j);
                if constexpr (P1::is_b(j)) f1.b[f] = rd.template b<f, 1>(b_stage(H));
                else f1.a[f] = rd.template a<f, H, 1>(as0);
            },
            [&](auto l_c) {
                ld.template issue_b<Cfg::HB + decltype(l_c)::value, MASKED>(a, smem, 1 - H, k1, wave);
            });
        wait_vmcnt<0>();
        lds_barrier();                            // B(t)
        const GF_LDS char* as1 = a_slot(t + 1);
        const GF_LDS char* es1 = e_slot(t + 1);
        const int eo1 = rd.eo((t + 1) & 7);
        const int k2 = (t + 2) * Cfg::BK, ja = (t + 3) >> 1, pe = (t + 1) & 7, je = (t + 9) >> 3;
        const uint32_t eoff = SppLoader<Cfg>::espan(pe, je, a.K);
        spp_step<Cfg, 0, Cfg::HB + Cfg::LA + Cfg::LE>(
            acc, f1, hi,
            [&](auto j_c) {
                constexpr int j = decltype(j_c)::value, f = P0::frag(j);
                if constexpr (j < P0::NE) e[f] = rd.template e<f>(es1, eo1);
                else if constexpr (P0::is_b(j)) f0.b[f] = rd.template b<f, 0>(b_stage(1 - H));
                else f0.a[f] = rd.template a<f, 1 - H, 0>(as1);
            },
            [&](auto l_c) {
                constexpr int l = decltype(l_c)::value;
                if constexpr (l < Cfg::HB)
                    ld.template issue_b<l, MASKED>(a, smem, H, k2, wave);
                else if constexpr (l < Cfg::HB + Cfg::LA)
                    ld.template issue_a<1 - H, l - Cfg::HB, MASKED>(a, smem, ja, wave);
                else
                    ld.template issue_e<l - Cfg::HB - Cfg::LA>(smem, pe, je, eoff, wave);
            });
    };
    // Steady state: every tile that tiles t and t+1 load (B up to t+3, A up
    // to t+5) lies wholly inside K.
    const int nfull = (nk > 0 && nk * Cfg::BK > a.K) ? nk - 1 : nk;
    int t = 0;
    for (; t + 6 <= nfull; t += 2) {
        tile(std::integral_constant<int, 0>{}, std::false_type{}, t);
        tile(std::integral_constant<int, 1>{}, std::false_type{}, t + 1);
    }
    for (; t < nk; t += 2) {
        tile(std::integral_constant<int, 0>{}, std::true_type{}, t);
        if (t + 1 < nk) tile(std::integral_constant<int, 1>{}, std::true_type{}, t + 1);
    }
    wait_vmcnt<0>();                              // no load may land after the epilogue starts
    sp_store_c<Cfg>(acc, a, smem, m0 + wm * Cfg::WTM, n0 + wn * Cfg::WTN, wave, lane, true);
#endif
}

template <class Cfg>
hipError_t launch_spp_gemm(const SpArgs& a, hipStream_t stream)
{
    auto kern = spp_gemm_kernel<Cfg>;
    static std::atomic<uint64_t> lds_opt_in{0};   // devices where the LDS size is opted into
    {
        const hipError_t err = opt_in_lds((const void*)kern, Cfg::LDS_BYTES, lds_opt_in, stream);
        if (err != hipSuccess) return err;
    }
    const int tiles = ceil_div(a.M, Cfg::BM) * ceil_div(a.N, Cfg::BN);
    hipLaunchKernelGGL(kern, dim3(tiles, 1, 1), dim3(Cfg::NT, 1, 1), Cfg::LDS_BYTES, stream, a);
    return hipGetLastError();
}

}  // namespace gf
