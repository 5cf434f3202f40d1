// inst_f32.hip -- fp32 kernel instantiations of the configuration table.
#include "../../include/gemm_mkl.h"
#include "configs.hpp"

namespace gmk {

void register_f32(std::vector<ConfigEntry> &t, DtypeKernels &k)
{
    typedef float T;
    const int d = GEMM_MKL_F32;
    t.push_back(make_entry<T, 64, 64, 2, 2, 0, 1, 2, 3>(d, 2, "f32 64x64 waves2x2 mfma16x16x4"));
    t.push_back(make_entry<T, 128, 128, 2, 2, 1, 2, 3>(d, 2, "f32 128x128 waves2x2 mfma16x16x4"));
    t.push_back(make_entry<T, 32, 64, 1, 2, 1, 2, 3>(d, 3, "f32 32x64 waves1x2 mfma16x16x4"));
    fill_dtype_kernels<T>(k);
}

}  // namespace gmk
