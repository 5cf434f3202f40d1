// inst_f32.hip -- fp32 kernel instantiations of the configuration table.
#include "../../include/gemm_mkl.h"
#include "configs.hpp"

namespace gmk {

void register_f32(std::vector<ConfigEntry> &t, DtypeKernels &k)
{
    typedef float T;
    const int d = GEMM_MKL_F32;
    //                  T  BM   BN   RB  waves MF  prefetch depths
    // fp32 tiles run one wave per SIMD: at depth 2 the ring does not cover the
    // memory latency.  Depth 3 measured 138.5 -> 132 us on 2048^3 and
    // 1061 -> 1031 us on 4096^3 (128x128), and 53.4 -> 40.7 us on
    // 512x2048x2048, 16.27 -> 15.97 us on 128x2048x2048 S=4 (64x64 mfma16).
    t.push_back(with_fixup<T, 128, 128, 128, 2, 2, 0, 32, 3>(with_grouped<T, 128, 128, 128, 2, 2, 0, 32, 2>(
        make_entry<T, 128, 128, 128, 2, 2, 32, 1, 2, 3, 4>(d, 3, 0.4f, "f32 128x128 k32 waves2x2 mfma32"))));
    t.push_back(with_grouped<T, 64, 64, 128, 2, 2, 0, 32, 2>(with_streamk<T, 64, 64, 128, 2, 2, 32, 2>(
        make_entry<T, 64, 64, 128, 2, 2, 32, 0, 1, 2, 3>(d, 2, 0.4f, "f32 64x64 k32 waves2x2 mfma32"))));
    // 16x16x4 MFMAs give each wave four independent accumulators where the
    // 32x32x2 form has one: 6-7% faster on every fp32 shape measured
    // (128x2048x2048 S=4 16.4 against 17.3 us, 1024x1024x4096 96.8 against
    // 104.0 us).  Its figure sits just above the 32x32 variant's so that it
    // wins their ties without changing any comparison with the 128x128 tile.
    t.push_back(with_fixup<T, 64, 64, 128, 2, 2, 0, 16, 3>(
        make_entry<T, 64, 64, 128, 2, 2, 16, 1, 2, 3, 4>(d, 3, 0.401f, "f32 64x64 k32 waves2x2 mfma16")));
    t.push_back(make_entry<T, 32, 64, 128, 1, 2, 16, 1, 2, 3>(d, 2, 0.25f, "f32 32x64 k32 waves1x2 mfma16"));
    // four producer waves beside the 64 x 64 tile's four MFMA waves: faster
    // than the same tile without them on every fp32 shape measured
    // (128x2048x2048 S=4 with the in-kernel fix-up 13.2-13.6 against
    // 14.9-15.3 us, 256x1024x1024 9.7 against 10.5, 2048^3 127 against 135,
    // 4096^3 985 against 1047 (1029 on 128 x 128))
    t.push_back(with_fixup<T, 64, 64, 128, 2, 2, 4, 16, 3>(
        make_entry_kp<T, 64, 64, 128, 2, 2, 1, 4, 16, 2, 3, 4>(d, 3, 0.43f, "f32 64x64 k32 waves2x2+4p mfma16")));
    fill_dtype_kernels<T>(k);
}

}  // namespace gmk
