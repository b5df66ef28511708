// One shard of the GEMM instantiations: configs whose index % kGemmShards
// equals GF_SHARD (set on the compiler command line).  Registration runs at
// library load, filling gf::g_gemm_table.
#include "configs.hpp"

#ifndef GF_SHARD
#error "compile with -DGF_SHARD=<index>"
#endif

namespace gf {
namespace {

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
        }
        register_from<I + 1>();
    }
}

const int registered = (register_from<0>(), 0);

}  // namespace
}  // namespace gf
