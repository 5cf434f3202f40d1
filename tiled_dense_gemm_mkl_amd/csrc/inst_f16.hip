// inst_f16.hip -- f16 kernel instantiations of the configuration table.
#include "../../include/gemm_mkl.h"
#include "configs.hpp"

namespace gmk {

void register_f16(std::vector<ConfigEntry> &t, DtypeKernels &k)
{
    typedef _Float16 T;
    const int d = GEMM_MKL_F16;
    //                  T  BM   BN   RB  waves MF  prefetch depths
    t.push_back(with_fixup<T, 256, 256, 64, 2, 2, 0, 32, 4>(with_grouped<T, 256, 256, 64, 2, 2, 0, 32, 4>(
        make_entry<T, 256, 256, 64, 2, 2, 32, 1, 2, 3, 4>(d, 4, 0.47f, "f16 256x256 k32 waves2x2 mfma32"))));
    t.push_back(make_entry<T, 256, 256, 64, 2, 4, 32, 2, 3, 4>(d, 3, 0.46f, "f16 256x256 k32 waves2x4 mfma32"));
    t.push_back(make_entry<T, 256, 256, 64, 4, 2, 32, 2, 3, 4>(d, 3, 0.46f, "f16 256x256 k32 waves4x2 mfma32"));
    t.push_back(with_grouped<T, 256, 256, 128, 2, 4, 0, 32, 1>(
        make_entry<T, 256, 256, 128, 2, 4, 32, 1>(d, 1, 0.48f, "f16 256x256 k64 waves2x4 mfma32")));
    t.push_back(make_entry<T, 256, 128, 128, 4, 2, 32, 1, 2>(d, 2, 0.42f, "f16 256x128 k64 waves4x2 mfma32"));
    t.push_back(make_entry<T, 256, 256, 128, 2, 2, 32, 1>(d, 1, 0.4f, "f16 256x256 k64 waves2x2 mfma32"));
    t.push_back(make_entry<T, 256, 128, 128, 2, 2, 32, 1, 2>(d, 2, 0.4f, "f16 256x128 k64 waves2x2 mfma32"));
    t.push_back(with_streamk<T, 128, 256, 128, 2, 2, 32, 2>(
        make_entry<T, 128, 256, 128, 2, 2, 32, 1, 2>(d, 2, 0.4f, "f16 128x256 k64 waves2x2 mfma32")));
    t.push_back(with_streamk<T, 128, 128, 128, 2, 2, 32, 2, 3>(
        make_entry<T, 128, 128, 128, 2, 2, 32, 0, 1, 2, 3>(d, 3, 0.4f, "f16 128x128 k64 waves2x2 mfma32")));
    // producer waves: NP extra waves issue every global->LDS load
    //                     T  BM   BN   RB  waves WK NP MF  prefetch depths
    t.push_back(with_fixup<T, 128, 128, 128, 2, 2, 4, 32, 4>(with_persistent<T, 128, 128, 128, 2, 2, 4, 32, 3>(
        with_grouped<T, 128, 128, 128, 2, 2, 4, 32, 4>(make_entry_kp<T, 128, 128, 128, 2, 2, 1, 4, 32, 2, 3, 4>(
            d, 4, 0.42f, "f16 128x128 k64 waves2x2+4p mfma32")))));
    t.push_back(make_entry_kp<T, 128, 128, 128, 2, 2, 1, 2, 32, 2>(d, 2, 0.41f, "f16 128x128 k64 waves2x2+2p mfma32"));
    // 96-column tiles, chosen only by configuration id (the bf16 table has the
    // measurements; f16 512 x 5632 x 2048: 17.6 vs 16.6 us on 128 x 128 + 4p)
    t.push_back(make_entry_kp<T, 128, 96, 128, 2, 2, 1, 4, 16, 2, 3, 4>(d, 4, 0.01f, "f16 128x96 k64 waves2x2+4p mfma16"));
    t.push_back(with_fixup<T, 128, 256, 128, 2, 2, 4, 32, 2>(
        make_entry_kp<T, 128, 256, 128, 2, 2, 1, 4, 32, 2>(d, 2, 0.46f, "f16 128x256 k64 waves2x2+4p mfma32")));
    t.push_back(with_fixup<T, 256, 128, 128, 2, 2, 4, 32, 2>(
        make_entry_kp<T, 256, 128, 128, 2, 2, 1, 4, 32, 2>(d, 2, 0.35f, "f16 256x128 k64 waves2x2+4p mfma32")));
    t.push_back(with_fixup<T, 128, 256, 64, 2, 2, 4, 32, 4>(
        make_entry_kp<T, 128, 256, 64, 2, 2, 1, 4, 32, 3, 4>(d, 4, 0.34f, "f16 128x256 k32 waves2x2+4p mfma32")));
    // k-groups: WK wave groups share each chunk's k-steps (fewer LDS reads per MFMA)
    //                    T  BM   BN   RB  waves WK MF  prefetch depths
    t.push_back(make_entry_k<T, 128, 128, 128, 2, 1, 2, 32, 2, 3>(d, 3, 0.4f, "f16 128x128 k64 waves2x1x2 mfma32"));
    t.push_back(make_entry_k<T, 128, 128, 128, 1, 2, 2, 32, 2, 3>(d, 3, 0.4f, "f16 128x128 k64 waves1x2x2 mfma32"));
    t.push_back(make_entry_k<T, 128, 128, 128, 2, 2, 2, 32, 2, 3>(d, 3, 0.4f, "f16 128x128 k64 waves2x2x2 mfma32"));
    t.push_back(with_grouped<T, 64, 64, 128, 2, 2, 0, 32, 2>(
        // one wave per SIMD: depth 3 covers the memory latency that depth 2
        // leaves exposed (bf16 1024x1024x4096 34.9 -> 20.4 us, 128x5632x2048
        // 12.0 -> 9.5 us, 512x2048x2048 12.2 -> 9.8 us)
        make_entry<T, 64, 64, 128, 2, 2, 32, 1, 2, 3>(d, 3, 0.24f, "f16 64x64 k64 waves2x2 mfma32")));
    t.push_back(make_entry<T, 128, 128, 128, 2, 2, 16, 2>(d, 2, 0.3f, "f16 128x128 k64 waves2x2 mfma16"));
    t.push_back(make_entry<T, 256, 256, 128, 2, 2, 16, 1>(d, 1, 0.4f, "f16 256x256 k64 waves2x2 mfma16"));
    t.push_back(make_entry<T, 256, 256, 128, 2, 4, 16, 1>(d, 1, 0.40f, "f16 256x256 k64 waves2x4 mfma16"));
    // 128 x 192 tiles with four producer waves at depth 3 (four 40 KB slots:
    // all of the LDS), for the K-split grids that put one workgroup on nearly
    // every compute unit (512 x 5632: 120 tiles, two splits, 240 workgroups).
    t.push_back(with_fixup<T, 128, 192, 128, 2, 2, 4, 32, 3>(
        make_entry_kp<T, 128, 192, 128, 2, 2, 1, 4, 32, 3>(d, 3, 0.30f, "f16 128x192 k64 waves2x2+4p mfma32")));
    // 32-wide K chunks with deep rings: a chunk is half the bytes of a 64-wide
    // one, so the same 160 KB of LDS keeps more of them (and more bytes) in
    // flight while the memory latency is covered
    t.push_back(make_entry_kp<T, 128, 128, 64, 2, 2, 1, 4, 32, 4, 6, 8>(d, 6, 0.30f, "f16 128x128 k32 waves2x2+4p mfma32"));
    t.push_back(with_fixup<T, 128, 192, 64, 2, 2, 4, 32, 6>(
        make_entry_kp<T, 128, 192, 64, 2, 2, 1, 4, 32, 4, 6, 7>(d, 6, 0.30f, "f16 128x192 k32 waves2x2+4p mfma32")));
    t.push_back(make_entry_kp<T, 64, 64, 128, 2, 2, 1, 4, 32, 2, 3, 4>(d, 3, 0.26f, "f16 64x64 k64 waves2x2+4p mfma32"));
    // The producer tiles on 16 x 16 MFMAs: faster than on 32 x 32 in every
    // interleaved A/B (graph replay, bf16 unless noted): 128 x 128 on
    // 512x5632x2048 15.05 us at depth 3 against 15.54 at depth 4 (fp16 16.17
    // against 16.36), 1024x5632x8192 95.9 against 97.2, 2048^3 17.5 against
    // 18.0; 128 x 256 on 1024x8192x2048 31.0 against 32.2, 1024x8192x8192
    // 101.8 against 109.4; 64 x 64 on 1024x1024x4096 15.6 against 17.2,
    // 512x2048x2048 9.20 against 9.51.  Their figures sit just above the
    // 32 x 32 variants', which keep the fix-up and grouped kernels.
    t.push_back(make_entry_kp<T, 128, 128, 128, 2, 2, 1, 4, 16, 3, 4>(d, 3, 0.43f, "f16 128x128 k64 waves2x2+4p mfma16"));
    t.push_back(make_entry_kp<T, 128, 256, 128, 2, 2, 1, 4, 16, 2>(d, 2, 0.47f, "f16 128x256 k64 waves2x2+4p mfma16"));
    t.push_back(make_entry_kp<T, 64, 64, 128, 2, 2, 1, 4, 16, 3>(d, 3, 0.27f, "f16 64x64 k64 waves2x2+4p mfma16"));
    fill_dtype_kernels<T>(k);
}

}  // namespace gmk
