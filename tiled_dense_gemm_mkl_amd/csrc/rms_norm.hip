// rms_norm.hip -- RMSNorm over the rows of a [rows][hidden] tensor, the row
// reduction that "一个可定制的编译器，用于为AI模型生成高效的融合GPU内核" lowers
// from torch.nn.RMSNorm to one GPU kernel (its Loop IR and generated kernel):
//
//   y[r][j] = (x[r][j] * rsqrt(sum_j' x[r][j']^2 * (1/hidden) + eps)) * weight[j]
//
// computed in fp32 whatever the storage type, with one rounding to the output
// type at the end.
//
// Design for gfx950 (the page's kernel stages a row in shared memory and reads
// it twice, one block of 256 threads per row):
//   - every row is read from HBM exactly once, into registers: a row is spread
//     over WPR waves of 64 lanes (1..16), each lane holding NV 16-byte vectors
//     (up to 8), so one wave moves NV KB per row with all loads in flight at
//     once;
//   - a wave sums its squares with DPP lane exchanges (every lane ends with the
//     same bits), the row's waves then add their sums through LDS in
//     ascending wave order: the result does not depend on timing;
//   - the weight (hidden elements, shared by all rows) stays in the L2 and
//     per-CU caches;
//   - x and y may be the same buffer (each lane writes only the elements it
//     read itself, after the row's sum is known).
// Rows whose size is not a multiple of 16 bytes, pointers that are not 16-byte
// aligned and rows longer than the largest vector variant take a general
// kernel: one 256-thread workgroup per row, element loads, x read twice.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "../../include/gemm_mkl.h"

namespace gmk {
void note_hip_error(hipError_t e);   // defined with the GEMM entry points
}

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

template <class T> struct Cvt;
template <> struct Cvt<float> {
    __device__ static __forceinline__ float to(float v) { return v; }
    __device__ static __forceinline__ float from(float v) { return v; }
};
template <> struct Cvt<__bf16> {
    __device__ static __forceinline__ float to(__bf16 v) { return (float)v; }
    __device__ static __forceinline__ __bf16 from(float v) { return (__bf16)v; }   // RNE
};
template <> struct Cvt<_Float16> {
    __device__ static __forceinline__ float to(_Float16 v) { return (float)v; }
    __device__ static __forceinline__ _Float16 from(float v)   // RNE
    {
        // Left visible, a product followed by this conversion is fused into
        // one mixed-precision multiply-add whose addend is +0, and a product
        // of -0 then comes out as +0.  The empty asm hands the conversion an
        // opaque fp32 value, so the product is rounded to fp32 and converted
        // with its sign.
        asm("" : "+v"(v));
        return (_Float16)v;
    }
};

// Sum over the 64 lanes of a wave, every lane ending with the same bits:
// DPP exchanges inside each row of 16 lanes (partner lane i^1, i^2, then the
// mirror of the half row and of the row; floating-point addition is
// commutative, so both partners of an exchange compute the same sum), then
// the four row sums are added in ascending row order.
template <int CTRL>
__device__ __forceinline__ float dpp_partner(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_partner<0xB1>(v);    // quad_perm [1,0,3,2]: lane i^1
    v += dpp_partner<0x4E>(v);    // quad_perm [2,3,0,1]: lane i^2
    v += dpp_partner<0x141>(v);   // row_half_mirror: the other quad of each 8 lanes
    v += dpp_partner<0x140>(v);   // row_mirror: the other half of each 16 lanes
    const int b = __builtin_bit_cast(int, v);
    return ((__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) +
             __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32))) +
           __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
}

constexpr int waves_per_block(int wpr) { return wpr < 4 ? 4 : wpr; }

// Cache policy of the row traffic: y is written once and not read again here,
// so its stores are non-temporal; x and the weight are read with the default
// policy.  Measured on MI355X against the other three combinations (both
// non-temporal, neither, loads only), this one was as fast or faster on every
// shape (16384 x 8192 bf16: 75 us against 87 us for both non-temporal).
constexpr int kStoreAux = 2;   // nt

// Buffer resource over [base, base + bytes): loads past the end return zero
// and stores past it are dropped, so ragged rows and rows past the last need
// no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Vector kernel: NV 16-byte vectors per lane, WPR waves per row.  Vector i of
// lane `lane` in wave k of a row covers elements [e, e + VE) with
// e = ((i * WPR + k) * 64 + lane) * VE, so every load instruction of a wave
// reads 1 KB of consecutive memory.  Requires hidden * sizeof(T) % 16 == 0 and
// 16-byte aligned x, weight and y; hidden <= NV * WPR * 64 * VE.
template <class T, int NV, int WPR>
__global__ __launch_bounds__(waves_per_block(WPR) * 64) void rms_norm_vec_kernel(
    const T *x, const T *__restrict__ w, T *y, int64_t rows, int H, float inv_h, float eps)
{
    constexpr int VE = 16 / (int)sizeof(T);
    constexpr int RPB = waves_per_block(WPR) / WPR;   // rows per workgroup
    typedef T vec_t __attribute__((ext_vector_type(VE)));
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int k = wave % WPR;
    const int64_t row = (int64_t)blockIdx.x * RPB + wave / WPR;
    const bool live = row < rows;   // the same for the whole wave
    const int row_bytes = live ? H * (int)sizeof(T) : 0;
    const __amdgpu_buffer_rsrc_t xr = row_rsrc(x + (live ? row : 0) * (int64_t)H, row_bytes);

    i32x4 v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i)
        v[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, ((i * WPR + k) * 64 + lane) * 16, 0, 0);
    // the weight's loads go out with the row's, before the reduction waits
    const bool has_w = w != nullptr;
    const __amdgpu_buffer_rsrc_t wr = row_rsrc(w, row_bytes);
    i32x4 wv[NV];
    if (has_w) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            wv[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, ((i * WPR + k) * 64 + lane) * 16, 0, 0);
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const vec_t t = __builtin_bit_cast(vec_t, v[i]);
#pragma unroll
        for (int q = 0; q < VE; ++q) {
            const float f = Cvt<T>::to(t[q]);
            ss += f * f;
        }
    }
    ss = wave_sum(ss);
    if constexpr (WPR > 1) {
        __shared__ float part[RPB * WPR];
        if (lane == 0) part[wave] = ss;
        __syncthreads();
        const int base = wave - k;
        ss = 0.0f;
#pragma unroll
        for (int j = 0; j < WPR; ++j) ss += part[base + j];
    }
    if (!live) return;
    const float r = rsqrtf(ss * inv_h + eps);
    const __amdgpu_buffer_rsrc_t yr = row_rsrc(y + row * (int64_t)H, row_bytes);
    if (has_w) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const vec_t xv = __builtin_bit_cast(vec_t, v[i]);
            const vec_t ww = __builtin_bit_cast(vec_t, wv[i]);
            vec_t o;
#pragma unroll
            for (int q = 0; q < VE; ++q) o[q] = Cvt<T>::from((Cvt<T>::to(xv[q]) * r) * Cvt<T>::to(ww[q]));
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o), yr,
                                                   ((i * WPR + k) * 64 + lane) * 16, 0, kStoreAux);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const vec_t xv = __builtin_bit_cast(vec_t, v[i]);
            vec_t o;
#pragma unroll
            for (int q = 0; q < VE; ++q) o[q] = Cvt<T>::from(Cvt<T>::to(xv[q]) * r);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, o), yr,
                                                   ((i * WPR + k) * 64 + lane) * 16, 0, kStoreAux);
        }
    }
}

// General kernel: any hidden size and element-aligned pointers.  One
// workgroup of 4 waves per row; x is read once for the sum and again for the
// output (the second read mostly hits the caches).
template <class T>
__global__ __launch_bounds__(256) void rms_norm_general_kernel(const T *x, const T *w, T *y, int64_t H, float inv_h,
                                                               float eps)
{
    const int64_t row = blockIdx.x;
    const T *xr = x + row * H;
    T *yr = y + row * H;
    float ss = 0.0f;
    for (int64_t j = threadIdx.x; j < H; j += 256) {
        const float f = Cvt<T>::to(xr[j]);
        ss += f * f;
    }
    ss = wave_sum(ss);
    __shared__ float part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    ss = ((part[0] + part[1]) + part[2]) + part[3];
    const float r = rsqrtf(ss * inv_h + eps);
    for (int64_t j = threadIdx.x; j < H; j += 256) {
        const float o = Cvt<T>::to(xr[j]) * r;
        yr[j] = Cvt<T>::from(w != nullptr ? o * Cvt<T>::to(w[j]) : o);
    }
}

typedef hipError_t (*RmsLaunch)(const void *, const void *, void *, int64_t, int64_t, float, float, hipStream_t);

// A launch covers at most 2^20 workgroups (well inside the 2^32 work-items a
// dispatch may hold); longer row ranges take several launches on the stream.
constexpr int64_t kMaxBlocksPerLaunch = int64_t(1) << 20;

template <class T, int NV, int WPR>
hipError_t launch_vec(const void *x, const void *w, void *y, int64_t rows, int64_t H, float inv_h, float eps,
                      hipStream_t s)
{
    constexpr int RPB = waves_per_block(WPR) / WPR;
    for (int64_t r0 = 0; r0 < rows; r0 += kMaxBlocksPerLaunch * RPB) {
        const int64_t n = rows - r0 < kMaxBlocksPerLaunch * RPB ? rows - r0 : kMaxBlocksPerLaunch * RPB;
        hipLaunchKernelGGL((rms_norm_vec_kernel<T, NV, WPR>), dim3((unsigned)((n + RPB - 1) / RPB)),
                           dim3(waves_per_block(WPR) * 64), 0, s, static_cast<const T *>(x) + r0 * H,
                           static_cast<const T *>(w), static_cast<T *>(y) + r0 * H, n, (int)H, inv_h, eps);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <class T>
hipError_t launch_general(const void *x, const void *w, void *y, int64_t rows, int64_t H, float inv_h, float eps,
                          hipStream_t s)
{
    for (int64_t r0 = 0; r0 < rows; r0 += kMaxBlocksPerLaunch) {
        const int64_t n = rows - r0 < kMaxBlocksPerLaunch ? rows - r0 : kMaxBlocksPerLaunch;
        hipLaunchKernelGGL((rms_norm_general_kernel<T>), dim3((unsigned)n), dim3(256), 0, s,
                           static_cast<const T *>(x) + r0 * H, static_cast<const T *>(w),
                           static_cast<T *>(y) + r0 * H, H, inv_h, eps);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

struct Variant {
    const char *name;
    int nv;     // 16-byte vectors per lane (0: general kernel)
    int wpr;    // waves per row
    RmsLaunch fn[3];   // by dtype: f32, f16, bf16
};

template <int NV, int WPR>
constexpr Variant vec_variant(const char *name)
{
    return Variant{name,
                   NV,
                   WPR,
                   {&launch_vec<float, NV, WPR>, &launch_vec<_Float16, NV, WPR>, &launch_vec<__bf16, NV, WPR>}};
}

// Variant 0 is the general kernel.  Variants 1..8 are the ladder the
// automatic choice climbs: each covers twice the row length of the one before
// (64 * NV * WPR vectors of 16 bytes), and the first whose coverage reaches
// hidden is taken, so at most half the lanes of a row's last vector step are
// idle.  At equal coverage the ladder takes the split measured fastest on
// MI355X (rows of 65536 x 2048 fp32 / 16384 x 8192 bf16: one vector per lane
// over 8 waves, four vectors over 4..16 waves).  The rest are the other splits,
// for sweeps.
const Variant kVariants[] = {
    {"general", 0, 0, {&launch_general<float>, &launch_general<_Float16>, &launch_general<__bf16>}},
    vec_variant<1, 1>("vec nv1 w1"),
    vec_variant<2, 1>("vec nv2 w1"),
    vec_variant<4, 1>("vec nv4 w1"),
    vec_variant<1, 8>("vec nv1 w8"),
    vec_variant<4, 4>("vec nv4 w4"),
    vec_variant<4, 8>("vec nv4 w8"),
    vec_variant<4, 16>("vec nv4 w16"),
    vec_variant<8, 16>("vec nv8 w16"),
    vec_variant<8, 1>("vec nv8 w1"),
    vec_variant<4, 2>("vec nv4 w2"),
    vec_variant<2, 4>("vec nv2 w4"),
    vec_variant<8, 2>("vec nv8 w2"),
    vec_variant<2, 8>("vec nv2 w8"),
    vec_variant<1, 16>("vec nv1 w16"),
    vec_variant<8, 4>("vec nv8 w4"),
    vec_variant<8, 8>("vec nv8 w8"),
};
constexpr int kNumVariants = (int)(sizeof(kVariants) / sizeof(kVariants[0]));
constexpr int kLadderEnd = 9;   // variants 1..8 form the automatic ladder

int elem_size(int dtype) { return dtype == GEMM_MKL_F32 ? 4 : 2; }

int64_t coverage(const Variant &v, int dtype) { return (int64_t)v.nv * v.wpr * 64 * (16 / elem_size(dtype)); }

bool vec_fits(const Variant &v, int64_t H, int dtype) { return v.nv == 0 || H <= coverage(v, dtype); }

// The variant the automatic choice takes: the first rung of the ladder that
// covers a row, when the vector kernels apply; else the general kernel.
int choose(int64_t H, int dtype, bool vec_ok)
{
    if (vec_ok)
        for (int i = 1; i < kLadderEnd; ++i)
            if (vec_fits(kVariants[i], H, dtype)) return i;
    return 0;
}

// True when the byte ranges [p, p + pn) and [q, q + qn) share a byte.
bool byte_overlap(const void *p, uint64_t pn, const void *q, uint64_t qn)
{
    if (pn == 0 || qn == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a <= b ? b - a < pn : a - b < qn;
}

int check(const void *x, const void *weight, const void *y, int64_t rows, int64_t H, float eps, int dtype,
          int variant, bool *vec_ok)
{
    if (dtype != GEMM_MKL_F32 && dtype != GEMM_MKL_F16 && dtype != GEMM_MKL_BF16)
        return GEMM_MKL_STATUS_UNSUPPORTED_DTYPE;
    if (rows < 0 || H < 0 || !(eps >= 0.0f) || std::isinf(eps)) return GEMM_MKL_STATUS_INVALID_VALUE;
    if (variant < -1 || variant >= kNumVariants) return GEMM_MKL_STATUS_INVALID_VALUE;
    const int64_t es = elem_size(dtype);
    if (H > INT32_MAX || (H > 0 && rows > INT64_MAX / H / es)) return GEMM_MKL_STATUS_INVALID_VALUE;
    auto al = [](const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
    if (rows > 0 && H > 0) {
        if (x == nullptr || y == nullptr) return GEMM_MKL_STATUS_INVALID_VALUE;
        if (!al(x, es) || !al(y, es) || !al(weight, es)) return GEMM_MKL_STATUS_INVALID_VALUE;
        // y may be x itself: a row's sum of squares is complete before any
        // of the row is written, and each element is then read by the thread
        // that overwrites it.  Any other byte that y shares with x or the
        // weight would let one row's output change another row's input.
        const uint64_t n = uint64_t(rows * H * es), wn = weight ? uint64_t(H * es) : 0;
        if ((y != x && byte_overlap(y, n, x, n)) || byte_overlap(y, n, weight, wn))
            return GEMM_MKL_STATUS_INVALID_VALUE;
    }
    *vec_ok = al(x, 16) && al(y, 16) && al(weight, 16) && (H * es) % 16 == 0;
    return GEMM_MKL_STATUS_OK;
}

bool log_enabled()
{
    static const bool on = [] {
        const char *v = std::getenv("GEMM_MKL_LOG");
        return v && *v && std::atoi(v) != 0;
    }();
    return on;
}

}  // namespace

extern "C" {

int gemm_mkl_rms_norm_ex(const void *x, const void *weight, void *y, int64_t rows, int64_t hidden, float eps,
                         int dtype, void *stream, int variant)
{
    bool vec_ok = false;
    const int st = check(x, weight, y, rows, hidden, eps, dtype, variant, &vec_ok);
    if (st != GEMM_MKL_STATUS_OK) return st;
    if (rows == 0 || hidden == 0) return GEMM_MKL_STATUS_OK;
    int v = variant;
    if (v < 0) {
        v = choose(hidden, dtype, vec_ok);
    } else if (kVariants[v].nv > 0 && !(vec_ok && vec_fits(kVariants[v], hidden, dtype))) {
        return GEMM_MKL_STATUS_NOT_AVAILABLE;
    }
    const float inv_h = (float)(1.0 / (double)hidden);
    if (log_enabled())
        std::fprintf(stderr, "gemm_mkl_rms_norm: rows=%lld hidden=%lld dtype=%d -> %s\n", (long long)rows,
                     (long long)hidden, dtype, kVariants[v].name);
    const hipError_t e =
        kVariants[v].fn[dtype](x, weight, y, rows, hidden, inv_h, eps, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        gmk::note_hip_error(e);
        return GEMM_MKL_STATUS_HIP_ERROR;
    }
    return GEMM_MKL_STATUS_OK;
}

int gemm_mkl_rms_norm(const void *x, const void *weight, void *y, int64_t rows, int64_t hidden, float eps, int dtype,
                      void *stream)
{
    return gemm_mkl_rms_norm_ex(x, weight, y, rows, hidden, eps, dtype, stream, -1);
}

int gemm_mkl_rms_norm_variant(int64_t rows, int64_t hidden, int dtype, int aligned)
{
    if (dtype != GEMM_MKL_F32 && dtype != GEMM_MKL_F16 && dtype != GEMM_MKL_BF16)
        return GEMM_MKL_STATUS_UNSUPPORTED_DTYPE;
    if (rows < 0 || hidden < 0 || hidden > INT32_MAX) return GEMM_MKL_STATUS_INVALID_VALUE;
    const bool vec_ok = aligned != 0 && (hidden * elem_size(dtype)) % 16 == 0;
    return choose(hidden, dtype, vec_ok);
}

int gemm_mkl_rms_norm_num_variants(void) { return kNumVariants; }

const char *gemm_mkl_rms_norm_variant_name(int variant)
{
    if (variant < 0 || variant >= kNumVariants) return nullptr;
    return kVariants[variant].name;
}

}  // extern "C"
