// 2:4 structured-sparse GEMM and compression: kernel instances and C-ABI
// entry points.  Validation runs on the host before any HIP call.
#include <stdint.h>

#include "../../include/gemvfp16.h"
#include "sparse_kernel.hpp"

namespace gf {
namespace {

constexpr int64_t kSpMaxElems = (int64_t(1) << 31) - 1;
constexpr int kSpDefaultPanel = 10;

bool sp_aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

typedef hipError_t (*SpLaunchFn)(const SpArgs&, hipStream_t);

struct SpDesc {
    int bm, bn, stages;
    SpLaunchFn fn;
};

template <int BM, int BN, int S>
constexpr SpDesc sp_desc()
{
    return SpDesc{BM, BN, S, &launch_sp_gemm<SpCfg<BM, BN, S>, true>};
}

// The paired form (stages = 0): two B stages, A_sparse in K-tile pairs,
// metadata eight K tiles at a time; half of each B tile's loads under the
// last MFMA step of the tile two before.
template <int BM, int BN, int S, int HB>
constexpr SpDesc spp_desc()
{
    static_assert(S == 0 && SpPairCfg<BM, BN, HB>::kValid, "invalid paired sparse config");
    return SpDesc{BM, BN, S, &launch_spp_gemm<SpPairCfg<BM, BN, HB>>};
}

// Compiled tile configs (the offline sweep times each of them).
const SpDesc kSpConfigs[] = {
    sp_desc<256, 256, 2>(), sp_desc<256, 256, 3>(),
    sp_desc<256, 128, 2>(), sp_desc<256, 128, 3>(), sp_desc<256, 128, 4>(),
    sp_desc<128, 256, 2>(), sp_desc<128, 256, 3>(),
    sp_desc<128, 128, 2>(), sp_desc<128, 128, 3>(), sp_desc<128, 128, 4>(),
    spp_desc<256, 256, 0, 4>(), spp_desc<256, 128, 0, 2>(), spp_desc<128, 256, 0, 4>(),
    spp_desc<128, 128, 0, 2>(),
};
constexpr int kNumSp = sizeof(kSpConfigs) / sizeof(kSpConfigs[0]);

static_assert(SpCfg<256, 256, 2>::kValid && SpCfg<256, 256, 3>::kValid && SpCfg<256, 128, 2>::kValid &&
                  SpCfg<256, 128, 3>::kValid && SpCfg<256, 128, 4>::kValid && SpCfg<128, 256, 2>::kValid &&
                  SpCfg<128, 256, 3>::kValid && SpCfg<128, 128, 2>::kValid && SpCfg<128, 128, 3>::kValid &&
                  SpCfg<128, 128, 4>::kValid,
              "every listed sparse config must be valid");

// Operands without the direct-to-LDS alignment take one register-staged kernel.
typedef SpCfg<128, 128, 2> SpFallbackCfg;

int find_sp(const gf_sp_cfg& c)
{
    for (int i = 0; i < kNumSp; ++i)
        if (kSpConfigs[i].bm == c.block_m && kSpConfigs[i].bn == c.block_n && kSpConfigs[i].stages == c.stages)
            return i;
    return -1;
}

// The largest tile that still gives every CU a workgroup: 256 x 256 with
// three stages; where only half-size tiles fill the CUs, 128 x 256 with
// three stages; else 128 x 128 with three stages.  The half-size case was
// timed side by side with B rotated through HBM, alternating batch by batch,
// at 2048 x 4096, 4096 x 2048, 3072 x 4096, 4096 x 3072, 1536 x 8192,
// 1024 x 8192 and 8192 x 1024 (K = 8192; 2048 x 4096 also at K = 4096 and
// 16384): 128 x 256 with three stages ran 7-36 % ahead of the paired form
// of 256 x 128, and ahead of or within 2 % of the other half-size tiles.
// Cache-warm sweeps had ranked the paired form first; with B streaming from
// HBM its single-line A loads no longer pay for its two-deep B pipeline.
gf_sp_cfg default_sp_cfg(int M, int N)
{
    gf_sp_cfg c;
    c.raster = 1;
    const int64_t t256 = (int64_t)ceil_div(M, 256) * ceil_div(N, 256);
    const int64_t t25612 = (int64_t)ceil_div(M, 256) * ceil_div(N, 128);
    if (t256 >= 256) { c.block_m = 256; c.block_n = 256; c.stages = 3; }
    else if (t25612 >= 256) { c.block_m = 128; c.block_n = 256; c.stages = 3; }
    else { c.block_m = 128; c.block_n = 128; c.stages = 3; }
    return c;
}

// Wave quantisation of the 256 x 256 tile (one workgroup per CU, so tiles
// run in rounds of 256): when the last round would be at most half full, the
// leading tile-rows that fill whole rounds run as one launch and the
// remaining rows (at most 1024) as a second launch with the tile the library
// picks for their size.  Returns the row count of the first part; M means no
// split.  A_sparse, E and C rows are contiguous, and every tile form issues
// the same sparse MFMAs over K in the same order, so the result does not
// depend on the split.
int sp_row_split(int M, int N, const gf_sp_cfg& c)
{
    constexpr int64_t kCus = 256, kMaxTailRows = 1024;
    if (c.block_m != 256 || c.block_n != 256) return M;
    const int64_t tn = ceil_div(N, 256), tiles = (int64_t)ceil_div(M, 256) * tn;
    const int64_t rounds = (tiles + kCus - 1) / kCus;
    if (rounds < 2 || tiles - kCus * (rounds - 1) > kCus / 2) return M;
    const int64_t m1 = (kCus * (rounds - 1) / tn) * 256;
    if (m1 < 256 || m1 >= M || M - m1 > kMaxTailRows) return M;
    return (int)m1;
}

int validate_sp(const void* Asp, const void* E, const void* B, const void* C, int M, int N, int K)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return GF_ERR_INVALID_ARG;
    if ((int64_t)M * K > kSpMaxElems || (int64_t)N * K > kSpMaxElems || (int64_t)M * N > kSpMaxElems)
        return GF_ERR_INVALID_ARG;
    if (M > 0 && K > 0 && (!Asp || !E || !sp_aligned(Asp, 2) || !sp_aligned(E, 2))) return GF_ERR_INVALID_ARG;
    if (N > 0 && K > 0 && (!B || !sp_aligned(B, 2))) return GF_ERR_INVALID_ARG;
    if (M > 0 && N > 0 && (!C || !sp_aligned(C, 2))) return GF_ERR_INVALID_ARG;
    return GF_OK;
}

int sp_impl(const void* Asp, const void* E, const void* B, void* C, int M, int N, int K, const gf_sp_cfg& cfg,
            hipStream_t stream)
{
    const int idx = find_sp(cfg);
    if (idx < 0) return GF_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return GF_OK;
    SpArgs a;
    a.Asp = (const uint16_t*)Asp;
    a.E = (const uint16_t*)E;
    a.B = (const uint16_t*)B;
    a.C = (uint16_t*)C;
    a.M = M; a.N = N; a.K = K;
    a.raster = cfg.raster <= 0 ? 0 : (cfg.raster == 1 ? kSpDefaultPanel : cfg.raster);
    const bool al = K % 32 == 0 && sp_aligned(Asp, 16) && sp_aligned(B, 16) && sp_aligned(E, 4);
    hipError_t e = al ? kSpConfigs[idx].fn(a, stream) : launch_sp_gemm<SpFallbackCfg, false>(a, stream);
    return e == hipSuccess ? GF_OK : GF_ERR_HIP;
}

}  // namespace
}  // namespace gf

using namespace gf;

extern "C" {

int sp24_compress_f16(const void* A, void* A_sparse, void* E, int M, int K, void* stream)
{
    if (M < 0 || K < 0 || K % 16 != 0 || (int64_t)M * K > kSpMaxElems) return GF_ERR_INVALID_ARG;
    if (M == 0 || K == 0) return GF_OK;
    if (!A || !A_sparse || !E || !sp_aligned(A, 2) || !sp_aligned(A_sparse, 2) || !sp_aligned(E, 2))
        return GF_ERR_INVALID_ARG;
    const size_t words = (size_t)M * (size_t)(K / 16);
    const int grid = (int)((words + 255) / 256 < 8192 ? (words + 255) / 256 : 8192);
    hipStream_t s = (hipStream_t)stream;
    if (sp_aligned(A, 16) && sp_aligned(A_sparse, 16))
        hipLaunchKernelGGL(sp24_compress_kernel, dim3(grid), dim3(256), 0, s, (const u32x4*)A, (u32x4*)A_sparse,
                           (uint16_t*)E, words);
    else
        hipLaunchKernelGGL(sp24_compress_kernel_u16, dim3(grid), dim3(256), 0, s, (const uint16_t*)A,
                           (uint16_t*)A_sparse, (uint16_t*)E, words);
    return hipGetLastError() == hipSuccess ? GF_OK : GF_ERR_HIP;
}

int gemm_sp_f16_nt_cfg(const void* A_sparse, const void* E, const void* B, void* C, int M, int N, int K,
                       const gf_sp_cfg* cfg, void* stream)
{
    const int v = validate_sp(A_sparse, E, B, C, M, N, K);
    if (v != GF_OK) return v;
    const gf_sp_cfg c = cfg ? *cfg : default_sp_cfg(M, N);
    const int m1 = cfg ? M : sp_row_split(M, N, c);
    if (m1 < M) {
        const int rc = sp_impl(A_sparse, E, B, C, m1, N, K, c, (hipStream_t)stream);
        if (rc != GF_OK) return rc;
        // row m1 of A_sparse starts m1 * K bytes in, of E m1 * K / 8 bytes, of C m1 * N * 2 bytes
        return sp_impl(static_cast<const char*>(A_sparse) + (size_t)m1 * K,
                       static_cast<const char*>(E) + (size_t)m1 * (K / 8), B,
                       static_cast<char*>(C) + (size_t)m1 * N * 2, M - m1, N, K, default_sp_cfg(M - m1, N),
                       (hipStream_t)stream);
    }
    return sp_impl(A_sparse, E, B, C, M, N, K, c, (hipStream_t)stream);
}

int gemm_sp_f16_nt(const void* A_sparse, const void* E, const void* B, void* C, int M, int N, int K,
                   void* stream)
{
    return gemm_sp_f16_nt_cfg(A_sparse, E, B, C, M, N, K, nullptr, stream);
}

int gf_sp_config_count(void) { return kNumSp; }

int gf_sp_config_get(int i, gf_sp_cfg* out)
{
    if (i < 0 || i >= kNumSp || !out) return GF_ERR_INVALID_ARG;
    out->block_m = kSpConfigs[i].bm;
    out->block_n = kSpConfigs[i].bn;
    out->stages = kSpConfigs[i].stages;
    out->raster = 1;
    return GF_OK;
}

int gf_sp_default_config(int M, int N, int K, gf_sp_cfg* out)
{
    if (!out || M < 0 || N < 0 || K < 0) return GF_ERR_INVALID_ARG;
    *out = default_sp_cfg(M, N);
    return GF_OK;
}

}  // extern "C"
