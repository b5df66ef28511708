// Skinny GEMM instantiations (every launch shape), registered at library
// load into gf::g_skinny_table.
#include "configs.hpp"
#include "skinny_kernel.hpp"

namespace gf {

SkinnyLaunchFn g_skinny_table[kNumSkinny] = {};

namespace {

template <int I>
void register_from()
{
    if constexpr (I < kNumSkinny) {
        constexpr SkinnyDesc d = kSkinnyConfigs[I];
        if constexpr (d.stages == 0)
            g_skinny_table[I] = &launch_skinny<d.blocks, d.unroll, d.waves>;
        else if constexpr (d.stages == 1)
            g_skinny_table[I] = &launch_skinny_vec<d.blocks, d.unroll, d.waves>;
        else if constexpr (d.stages < 0)
            g_skinny_table[I] = &launch_skinny_split<d.blocks, d.unroll, d.waves>;
        else if constexpr (SkinnyLdsCfg<d.blocks, d.stages, d.waves>::kValid)
            g_skinny_table[I] = &launch_skinny_lds<d.blocks, d.stages, d.waves>;
        register_from<I + 1>();
    }
}

const int registered = (register_from<0>(), 0);

}  // namespace
}  // namespace gf
