// configs.hpp -- the kernel configuration table shared by the host dispatcher
// and the per-dtype instantiation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "gemm_kernels.hpp"

namespace gmk {

constexpr int kMaxPrefetch = 8;   // prefetch_stages 0..8 (ring of 1..9 LDS slots)
constexpr int kModes = 4;         // identity, relu, silu, split-K partial

typedef hipError_t (*TileLaunchFn)(const TileParams &p, int grid, hipStream_t stream);
typedef hipError_t (*StreamKLaunchFn)(const StreamKParams &p, int grid, hipStream_t stream);
typedef hipError_t (*GroupedLaunchFn)(const GroupedParams &p, int grid, hipStream_t stream);
typedef hipError_t (*FixupLaunchFn)(const FixupParams &p, int grid, hipStream_t stream);
typedef hipError_t (*ReduceLaunchFn)(const float *W, void *C, int64_t total, int split, hipStream_t stream);
typedef hipError_t (*GeneralLaunchFn)(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K,
                                      int64_t L, hipStream_t stream);
typedef hipError_t (*PackLaunchFn)(const void *src, void *dst, int64_t rows, int64_t K, int64_t Kp,
                                   hipStream_t stream);

struct ConfigEntry {
    int dtype;             // GEMM_MKL_F32 / F16 / BF16
    int bm, bn;            // output tile
    int rb;                // bytes of K per row in one chunk (64 or 128)
    int mf;                // MFMA block edge (16 or 32)
    int waves_m, waves_n;  // wave grid (64 lanes each)
    int waves_k;           // wave groups splitting each chunk's k-steps
    int producers;         // extra waves that only issue the global->LDS loads
    int default_p;         // prefetch_stages used when not forced
    float eff;             // measured fraction of the dtype's MFMA peak on large problems
    const char *name;
    TileLaunchFn fn[kMaxPrefetch + 1][kModes];  // null where not instantiated
    StreamKLaunchFn sk[kMaxPrefetch + 1][3];    // stream-K by epilogue, null where not instantiated
    GroupedLaunchFn grouped[3];                 // grouped GEMM by epilogue (depth grouped_p), or null
    int grouped_p;
    TileLaunchFn persist[3];                    // persistent grid by epilogue (depth persist_p), or null
    int persist_p;
    FixupLaunchFn fixup[3];                     // split-K with the in-kernel fix-up (default_p), or null
};

struct DtypeKernels {
    ReduceLaunchFn reduce[3];    // by epilogue
    GeneralLaunchFn general[3];  // by epilogue
    PackLaunchFn pack;           // operand rows into 16-byte aligned, zero-padded rows
};

// Filled by the instantiation units (one per dtype).
void register_f32(std::vector<ConfigEntry> &table, DtypeKernels &k);
void register_f16(std::vector<ConfigEntry> &table, DtypeKernels &k);
void register_bf16(std::vector<ConfigEntry> &table, DtypeKernels &k);

// ---------------------------------------------------------------- helpers for the units

template <class T, int BM, int BN, int RB, int WMW, int WNW, int MF, int P, int MODE, int WK, int NP>
hipError_t launch_tile(const TileParams &p, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_tile_kernel<T, BM, BN, RB, WMW, WNW, MF, P, MODE, WK, NP>), dim3(grid),
                       dim3((WMW * WNW * WK + NP) * 64), 0, stream, p);
    return hipGetLastError();
}

template <class T, int BM, int BN, int RB, int WMW, int WNW, int MF, int P, int MODE>
hipError_t launch_streamk(const StreamKParams &p, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_streamk_kernel<T, BM, BN, RB, WMW, WNW, MF, P, MODE>), dim3(grid),
                       dim3(WMW * WNW * 64), 0, stream, p);
    return hipGetLastError();
}

template <class T, int BM, int BN, int RB, int WMW, int WNW, int MF, int P, int MODE, int NP>
hipError_t launch_grouped(const GroupedParams &p, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_grouped_kernel<T, BM, BN, RB, WMW, WNW, MF, P, MODE, NP>), dim3(grid),
                       dim3((WMW * WNW + NP) * 64), 0, stream, p);
    return hipGetLastError();
}

// Adds the grouped-GEMM kernels (prefetch depth P, NP producer waves) to an
// entry made by make_entry_kp with the same tile and wave grid.
template <class T, int BM, int BN, int RB, int WMW, int WNW, int NP, int MF, int P>
ConfigEntry with_grouped(ConfigEntry e)
{
    static_assert(P >= 2 || NP == 0, "producer waves need a ring of at least 3 slots");
    e.grouped[MODE_IDENTITY] = &launch_grouped<T, BM, BN, RB, WMW, WNW, MF, P, MODE_IDENTITY, NP>;
    e.grouped[MODE_RELU] = &launch_grouped<T, BM, BN, RB, WMW, WNW, MF, P, MODE_RELU, NP>;
    e.grouped[MODE_SILU] = &launch_grouped<T, BM, BN, RB, WMW, WNW, MF, P, MODE_SILU, NP>;
    e.grouped_p = P;
    return e;
}

template <class T, int BM, int BN, int RB, int WMW, int WNW, int MF, int P, int MODE, int NP>
hipError_t launch_persistent(const TileParams &p, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_persistent_kernel<T, BM, BN, RB, WMW, WNW, MF, P, MODE, NP>), dim3(grid),
                       dim3((WMW * WNW + NP) * 64), 0, stream, p);
    return hipGetLastError();
}

// Adds the persistent-grid kernels (prefetch depth P, NP producer waves) to an
// entry made by make_entry_kp with the same tile and wave grid.
template <class T, int BM, int BN, int RB, int WMW, int WNW, int NP, int MF, int P>
ConfigEntry with_persistent(ConfigEntry e)
{
    static_assert(NP > 0 && P >= 2, "the persistent ring uses producer waves");
    e.persist[MODE_IDENTITY] = &launch_persistent<T, BM, BN, RB, WMW, WNW, MF, P, MODE_IDENTITY, NP>;
    e.persist[MODE_RELU] = &launch_persistent<T, BM, BN, RB, WMW, WNW, MF, P, MODE_RELU, NP>;
    e.persist[MODE_SILU] = &launch_persistent<T, BM, BN, RB, WMW, WNW, MF, P, MODE_SILU, NP>;
    e.persist_p = P;
    return e;
}

template <class T, int BM, int BN, int RB, int WMW, int WNW, int MF, int P, int MODE, int NP>
hipError_t launch_fixup(const FixupParams &p, int grid, hipStream_t stream)
{
    hipLaunchKernelGGL((gemm_fixup_kernel<T, BM, BN, RB, WMW, WNW, MF, P, MODE, NP>), dim3(grid),
                       dim3((WMW * WNW + NP) * 64), 0, stream, p);
    return hipGetLastError();
}

// Adds the split-K kernels with the in-kernel fix-up (prefetch depth P, the
// entry's default, NP producer waves) to an entry made by make_entry_kp with
// the same tile and wave grid.
template <class T, int BM, int BN, int RB, int WMW, int WNW, int NP, int MF, int P>
ConfigEntry with_fixup(ConfigEntry e)
{
    e.fixup[MODE_IDENTITY] = &launch_fixup<T, BM, BN, RB, WMW, WNW, MF, P, MODE_IDENTITY, NP>;
    e.fixup[MODE_RELU] = &launch_fixup<T, BM, BN, RB, WMW, WNW, MF, P, MODE_RELU, NP>;
    e.fixup[MODE_SILU] = &launch_fixup<T, BM, BN, RB, WMW, WNW, MF, P, MODE_SILU, NP>;
    return e;
}

// Stream-K variants of a configuration for prefetch depth P.
template <class T, int BM, int BN, int RB, int WMW, int WNW, int MF, int P>
void fill_streamk(ConfigEntry &e)
{
    static_assert(P >= 0 && P <= kMaxPrefetch, "prefetch depth outside the launch table");
    e.sk[P][MODE_IDENTITY] = &launch_streamk<T, BM, BN, RB, WMW, WNW, MF, P, MODE_IDENTITY>;
    e.sk[P][MODE_RELU] = &launch_streamk<T, BM, BN, RB, WMW, WNW, MF, P, MODE_RELU>;
    e.sk[P][MODE_SILU] = &launch_streamk<T, BM, BN, RB, WMW, WNW, MF, P, MODE_SILU>;
}

template <class T, int BM, int BN, int RB, int WMW, int WNW, int WK, int NP, int MF, int P>
void fill_prefetch(ConfigEntry &e)
{
    static_assert(P >= 0 && P <= kMaxPrefetch, "prefetch depth outside the launch table");
    e.fn[P][MODE_IDENTITY] = &launch_tile<T, BM, BN, RB, WMW, WNW, MF, P, MODE_IDENTITY, WK, NP>;
    e.fn[P][MODE_RELU] = &launch_tile<T, BM, BN, RB, WMW, WNW, MF, P, MODE_RELU, WK, NP>;
    e.fn[P][MODE_SILU] = &launch_tile<T, BM, BN, RB, WMW, WNW, MF, P, MODE_SILU, WK, NP>;
    e.fn[P][MODE_PARTIAL] = &launch_tile<T, BM, BN, RB, WMW, WNW, MF, P, MODE_PARTIAL, WK, NP>;
}

// A configuration: tile BM x BN, RB bytes of K per row and chunk, a WMW x WNW
// wave grid repeated over WK k-groups plus NP producer waves, MFMA edge MF,
// instantiated for prefetch depths Ps.
template <class T, int BM, int BN, int RB, int WMW, int WNW, int WK, int NP, int MF, int... Ps>
ConfigEntry make_entry_kp(int dtype, int default_p, float eff, const char *name)
{
    ConfigEntry e{};
    e.eff = eff;
    e.dtype = dtype;
    e.bm = BM;
    e.bn = BN;
    e.rb = RB;
    e.mf = MF;
    e.waves_m = WMW;
    e.waves_n = WNW;
    e.waves_k = WK;
    e.producers = NP;
    e.default_p = default_p;
    e.name = name;
    (fill_prefetch<T, BM, BN, RB, WMW, WNW, WK, NP, MF, Ps>(e), ...);
    return e;
}

template <class T, int BM, int BN, int RB, int WMW, int WNW, int WK, int MF, int... Ps>
ConfigEntry make_entry_k(int dtype, int default_p, float eff, const char *name)
{
    return make_entry_kp<T, BM, BN, RB, WMW, WNW, WK, 0, MF, Ps...>(dtype, default_p, eff, name);
}

template <class T, int BM, int BN, int RB, int WMW, int WNW, int MF, int... Ps>
ConfigEntry make_entry(int dtype, int default_p, float eff, const char *name)
{
    return make_entry_kp<T, BM, BN, RB, WMW, WNW, 1, 0, MF, Ps...>(dtype, default_p, eff, name);
}

// Adds stream-K variants (prefetch depths Ps) to an entry made by make_entry.
template <class T, int BM, int BN, int RB, int WMW, int WNW, int MF, int... Ps>
ConfigEntry with_streamk(ConfigEntry e)
{
    (fill_streamk<T, BM, BN, RB, WMW, WNW, MF, Ps>(e), ...);
    return e;
}

template <class T, int MODE>
hipError_t launch_reduce(const float *W, void *C, int64_t total, int split, hipStream_t stream)
{
    int64_t per_thread = (total % 4 == 0) ? 4 : 1;
    int64_t blocks = (total / per_thread + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((splitk_reduce_kernel<T, MODE>), dim3((unsigned)blocks), dim3(256), 0, stream, W,
                       reinterpret_cast<T *>(C), total, split);
    return hipGetLastError();
}

template <class T, int MODE>
hipError_t launch_general(const void *A, const void *B, void *C, int64_t M, int64_t N, int64_t K, int64_t L,
                          hipStream_t stream)
{
    const int64_t tm = (M + 63) / 64, tn = (N + 63) / 64;
    hipLaunchKernelGGL((gemm_general_kernel<T, MODE>), dim3((unsigned)(tm * tn * L)), dim3(256), 0, stream,
                       reinterpret_cast<const T *>(A), reinterpret_cast<const T *>(B), reinterpret_cast<T *>(C),
                       M, N, K, (int32_t)tm, (int32_t)tn);
    return hipGetLastError();
}

template <class T>
hipError_t launch_pack(const void *src, void *dst, int64_t rows, int64_t K, int64_t Kp, hipStream_t stream)
{
    const int64_t blocks = rows < 65536 ? rows : 65536;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL((pack_rows_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const T *>(src), reinterpret_cast<T *>(dst), rows, K, Kp);
    return hipGetLastError();
}

template <class T>
void fill_dtype_kernels(DtypeKernels &k)
{
    k.pack = &launch_pack<T>;
    k.reduce[0] = &launch_reduce<T, MODE_IDENTITY>;
    k.reduce[1] = &launch_reduce<T, MODE_RELU>;
    k.reduce[2] = &launch_reduce<T, MODE_SILU>;
    k.general[0] = &launch_general<T, MODE_IDENTITY>;
    k.general[1] = &launch_general<T, MODE_RELU>;
    k.general[2] = &launch_general<T, MODE_SILU>;
}

}  // namespace gmk
