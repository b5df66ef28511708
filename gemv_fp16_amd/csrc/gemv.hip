// GEMV instantiations (all launch shapes, aligned and masked), registered at
// library load into gf::g_gemv_table.
#include "configs.hpp"
#include "gemv_kernel.hpp"

namespace gf {

GemvLaunchFn g_gemv_table[kNumGemv][2] = {};

namespace {

template <int I>
void register_from()
{
    if constexpr (I < kNumGemv) {
        constexpr GemvDesc d = kGemvConfigs[I];
        g_gemv_table[I][1] = &launch_gemv<d.rows, d.unroll, d.waves, true>;
        g_gemv_table[I][0] = &launch_gemv<d.rows, d.unroll, d.waves, false>;
        register_from<I + 1>();
    }
}

const int registered = (register_from<0>(), 0);

}  // namespace
}  // namespace gf
