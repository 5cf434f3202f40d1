// inst_bf16.hip -- bf16 kernel instantiations of the configuration table.
#include "../../include/gemm_mkl.h"
#include "configs.hpp"

namespace gmk {

void register_bf16(std::vector<ConfigEntry> &t, DtypeKernels &k)
{
    typedef __bf16 T;
    const int d = GEMM_MKL_BF16;
    t.push_back(make_entry<T, 128, 128, 2, 2, 0, 1, 2, 3>(d, 2, "bf16 128x128 waves2x2 mfma16x16x32"));
    t.push_back(make_entry<T, 256, 128, 2, 2, 1, 2>(d, 2, "bf16 256x128 waves2x2 mfma16x16x32"));
    t.push_back(make_entry<T, 128, 256, 2, 2, 1, 2>(d, 2, "bf16 128x256 waves2x2 mfma16x16x32"));
    t.push_back(make_entry<T, 64, 64, 2, 2, 1, 2, 3>(d, 3, "bf16 64x64 waves2x2 mfma16x16x32"));
    fill_dtype_kernels<T>(k);
}

}  // namespace gmk
