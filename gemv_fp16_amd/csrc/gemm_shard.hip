// One shard of the GEMM instantiations: configs whose index % kGemmShards
// equals GF_SHARD (set on the compiler command line).  Registration runs at
// library load, filling gf::g_gemm_table.
#include "configs.hpp"

#ifndef GF_SHARD
#error "compile with -DGF_SHARD=<index>"
#endif

namespace gf {
namespace {

// fp16 GEMM of config I with operand layouts LAY = a_kmajor * 2 + b_kmajor.
template <int I, int LAY>
void register_layout()
{
    constexpr GemmDesc d = kGemmConfigs[I];
    typedef GemmCfg<d.bm, d.bn, d.bk, d.stages, d.threads, d.sched, LAY / 2, LAY % 2> CL;
    if constexpr (CL::kValid) {
        g_gemm_layout_table[I][LAY][1] = &launch_gemm<CL, EPI_F16, true>;
        g_gemm_layout_table[I][LAY][0] = &launch_gemm<CL, EPI_F16, false>;
    }
}

template <int I>
void register_from()
{
    if constexpr (I < kNumGemm) {
        if constexpr (I % kGemmShards == GF_SHARD) {
            constexpr GemmDesc d = kGemmConfigs[I];
            typedef GemmCfg<d.bm, d.bn, d.bk, d.stages, d.threads, d.sched> C;
            if constexpr (C::kValid) {
                g_gemm_table[I][EPI_F16 * 2 + 1] = &launch_gemm<C, EPI_F16, true>;
                if constexpr (d.core) {
                    g_gemm_table[I][EPI_F16 * 2 + 0] = &launch_gemm<C, EPI_F16, false>;
                    g_gemm_table[I][EPI_F32_ATOMIC * 2 + 1] = &launch_gemm<C, EPI_F32_ATOMIC, true>;
                    g_gemm_table[I][EPI_F32_ATOMIC * 2 + 0] = &launch_gemm<C, EPI_F32_ATOMIC, false>;
                    g_gemm_table[I][EPI_F32_STORE * 2 + 1] = &launch_gemm<C, EPI_F32_STORE, true>;
                    g_gemm_table[I][EPI_F32_STORE * 2 + 0] = &launch_gemm<C, EPI_F32_STORE, false>;
                }
            }
            if constexpr (has_layouts(d)) {
                register_layout<I, 1>();
                register_layout<I, 2>();
                register_layout<I, 3>();
            }
        }
        register_from<I + 1>();
    }
}

const int registered = (register_from<0>(), 0);

}  // namespace
}  // namespace gf
