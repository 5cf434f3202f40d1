// gemm_kernels.hpp -- device code of the gfx950 (CDNA4) tiled dense GEMM.
//
//   C[l][m][n] = epilogue( sum_k A[l][m][k] * B[l][n][k] )
//
// A is [L][M][K], B is [L][N][K] (K contiguous), C is [L][M][N]; the modes are
// those of the persistent dense GEMM on "深入解析 CUTLASS CuTe DSL 的 JIT 函数参数生成机制"
// (section 2.3).  The hot path of one workgroup:
//
//   1. tile mapping: workgroup id -> (batch l, split s, BM x BN output tile),
//      remapped so that consecutive tiles run on the same XCD (shared L2);
//      the output-tile-to-workgroup lift is the tileify / blockify_launch step
//      of "一个可定制的编译器，用于为AI模型生成高效的融合GPU内核" (its Tile-IR pass list).
//   2. K chunking: K is cut into chunks of 128 bytes per row (BK = 64 for
//      16-bit types, 32 for fp32); chunks are the "K-outer" loop and the
//      64-byte MFMA k-steps inside a chunk the "K-inner" loop (chunk_matmul_k
//      in the same list).  With split-K, ranges of chunks become a grid
//      dimension (split_matmul_k).
//   3. LDS staging: every chunk of the A and B tiles is copied to LDS by
//      direct global->LDS buffer loads (16 bytes a lane), in a row-major
//      [rows][128 B] layout whose 16-byte columns are XOR-swizzled by the row
//      index, so that the MFMA operand reads are free of bank conflicts
//      (stage_inputs / split_inner_for_swizzle / pad_smem in the list above).
//   4. A ring of prefetch_stages + 1 LDS slots: the prologue issues chunks
//      0..P-1; iteration i waits for chunk i, then issues chunk i+P into the
//      slot that chunk i-1 used, then computes on chunk i.  This is the
//      manual software pipeline of section 3 of "CUTLASS CuTe DSL 控制流编程指南"
//      (prefetch loop, then a main loop that prefetches i + prefetch_stages
//      while it uses slot i mod stages).  P = 0 is load-then-use.
//   5. MFMA mainloop with fp32 accumulators (v_mfma_f32_16x16x32_{bf16,f16},
//      v_mfma_f32_16x16x4_f32); the operands are swapped (B tile as the MFMA's
//      first operand) so that each lane ends up owning 4 consecutive n.
//   6. Epilogue fused at compile time (identity / ReLU / SiLU, sections 2.3
//      and 7 of the two CuTe DSL pages) on the fp32 sum, then one rounding to
//      the output type; or, for split-K, an fp32 partial tile that the reduce
//      kernel sums in ascending split order before the same epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gmk {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

enum Mode { MODE_IDENTITY = 0, MODE_RELU = 1, MODE_SILU = 2, MODE_PARTIAL = 3 };

// Bytes of one staged row of a chunk, and of one MFMA k-step per row.
constexpr int kRowBytes = 128;
constexpr int kStepBytes = 64;
constexpr int kStepsPerChunk = kRowBytes / kStepBytes;
// A voffset at or above every buffer's num_records: the load returns zeros.
constexpr uint32_t kOutOfRange = 0x80000000u;

struct TileParams {
    const void *A;
    const void *B;
    void *C;          // output (modes 0..2) or fp32 workspace [S][L][M][N] (partial)
    int64_t M, N, K, L;
    int32_t tiles_m, tiles_n;
    int32_t split;            // S
    int32_t chunks_per_split; // chunks of kRowBytes per split (the last may be short)
    int32_t total_chunks;     // ceil(K * elem / kRowBytes)
};

// ------------------------------------------------------------------ epilogue

template <int MODE>
__device__ __forceinline__ float apply_epilogue(float x)
{
    if constexpr (MODE == MODE_RELU) {
        return x > 0.0f ? x : 0.0f;          // where(x > 0, x, 0): -0 and NaN give +0
    } else if constexpr (MODE == MODE_SILU) {
        return x / (1.0f + expf(-x));        // x * sigmoid(x)
    } else {
        return x;
    }
}

// ------------------------------------------------------------------ element types

template <class T> struct Elem;

template <> struct Elem<float> {
    static constexpr int bytes = 4;
    __device__ static __forceinline__ f32x4 mfma_step(i32x4 a, i32x4 b, f32x4 acc)
    {
        // one 16-byte read holds 4 consecutive k of a row: four 16x16x4 MFMAs,
        // MFMA j taking component j on both operands (same k on both sides)
        f32x4v av = __builtin_bit_cast(f32x4v, a);
        f32x4v bv = __builtin_bit_cast(f32x4v, b);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bv[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], bv[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], bv[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[3], bv[3], acc, 0, 0, 0);
        return acc;
    }
    __device__ static __forceinline__ float from_f32(float x) { return x; }
    __device__ static __forceinline__ float to_f32(float x) { return x; }
    __device__ static __forceinline__ void store4(float *p, float a, float b, float c, float d)
    {
        f32x4v v = {a, b, c, d};
        *reinterpret_cast<f32x4v *>(p) = v;
    }
};

template <> struct Elem<__bf16> {
    static constexpr int bytes = 2;
    __device__ static __forceinline__ f32x4 mfma_step(i32x4 a, i32x4 b, f32x4 acc)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ __bf16 from_f32(float x) { return (__bf16)x; }  // RNE
    __device__ static __forceinline__ float to_f32(__bf16 x) { return (float)x; }
    __device__ static __forceinline__ void store4(__bf16 *p, float a, float b, float c, float d)
    {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
        *reinterpret_cast<bf16x4 *>(p) = v;
    }
};

template <> struct Elem<_Float16> {
    static constexpr int bytes = 2;
    __device__ static __forceinline__ f32x4 mfma_step(i32x4 a, i32x4 b, f32x4 acc)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
    }
    __device__ static __forceinline__ _Float16 from_f32(float x) { return (_Float16)x; }  // RNE
    __device__ static __forceinline__ float to_f32(_Float16 x) { return (float)x; }
    __device__ static __forceinline__ void store4(_Float16 *p, float a, float b, float c, float d)
    {
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        f16x4 v = {(_Float16)a, (_Float16)b, (_Float16)c, (_Float16)d};
        *reinterpret_cast<f16x4 *>(p) = v;
    }
};

// ------------------------------------------------------------------ low-level helpers

// Buffer resource for raw (unswizzled) addressing; out-of-range reads return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t num_records)
{
    uint64_t b = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
    r[3] = 0x00020000;                                               // gfx9 data format word
    return r;
}

// One direct global->LDS load of 16 bytes per lane: lane t writes LDS bytes
// [lds_base + 16 t, lds_base + 16 t + 16).  The LDS base goes in M0.  It is
// written as inline asm so that the compiler does not add conservative waits
// for it; the ring below waits on vmcnt explicitly.  A write of M0 needs one
// wait state before an LDS-DMA instruction reads it, hence the s_nop.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voffset, uint32_t soffset)
{
    asm volatile("s_mov_b32 m0, %0\n\t"
                 "s_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_base), "v"(voffset), "s"(rsrc), "s"(soffset)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Workgroup barrier that first drains this wave's LDS reads.  No vmcnt wait:
// prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)reinterpret_cast<uintptr_t>(p);
}

// XOR swizzle of the 16-byte column of a 128-byte LDS row: keeps the 16 rows
// read by one 16-lane MFMA operand group on distinct banks.
__device__ __forceinline__ int swz(int row)
{
    return (row & 7) ^ ((row >> 3) & 1);
}

// Workgroup id -> logical tile id.  Hardware dispatches consecutive workgroup
// ids round-robin over the 8 XCDs; this gives each XCD a contiguous range of
// logical ids so that tiles sharing A rows or B columns share one L2.
__device__ __forceinline__ int xcd_remap(int wg, int grid)
{
    constexpr int kXcd = 8;
    int per = grid / kXcd;            // full rounds
    int full = per * kXcd;
    if (wg >= full) return wg;        // the ragged last round keeps its ids
    return (wg % kXcd) * per + wg / kXcd;
}

// ------------------------------------------------------------------ the tiled kernel

template <class T, int BM, int BN, int WAVES_M, int WAVES_N, int P, int MODE>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void gemm_tile_kernel(TileParams p)
{
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int ES = Elem<T>::bytes;
    constexpr int WTM = BM / WAVES_M;
    constexpr int WTN = BN / WAVES_N;
    constexpr int FM = WTM / 16;
    constexpr int FN = WTN / 16;
    constexpr int SLOTS = P + 1;
    constexpr int SLOT_BYTES = (BM + BN) * kRowBytes;
    constexpr int A_GROUPS = BM / 8;              // 8 rows x 128 B = one wave load
    constexpr int B_GROUPS = BN / 8;
    constexpr int A_LOADS = A_GROUPS / NW;        // loads per wave per chunk
    constexpr int B_LOADS = B_GROUPS / NW;
    constexpr int LOADS = A_LOADS + B_LOADS;
    static_assert(BM % (16 * WAVES_M) == 0 && BN % (16 * WAVES_N) == 0, "wave tile");
    static_assert(A_GROUPS % NW == 0 && B_GROUPS % NW == 0, "load split");
    static_assert(SLOTS * SLOT_BYTES <= 160 * 1024, "LDS budget of a gfx950 workgroup");
    static_assert(LOADS * (P > 0 ? P : 1) < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char smem[SLOTS * SLOT_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // ---- tile mapping: [l][s][tile_n][tile_m], tile_m fastest
    const int grid = gridDim.x;
    int t = xcd_remap(blockIdx.x, grid);
    const int tm = t % p.tiles_m;
    t /= p.tiles_m;
    const int tn = t % p.tiles_n;
    t /= p.tiles_n;
    const int s = t % p.split;
    const int l = t / p.split;

    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    const int64_t K = p.K;
    const int chunk0 = s * p.chunks_per_split;
    int nk = p.total_chunks - chunk0;
    if (nk > p.chunks_per_split) nk = p.chunks_per_split;
    if (nk < 0) nk = 0;

    // ---- buffer resources anchored at the tile's first row
    const T *Ab = reinterpret_cast<const T *>(p.A) + ((int64_t)l * p.M + m0) * K;
    const T *Bb = reinterpret_cast<const T *>(p.B) + ((int64_t)l * p.N + n0) * K;
    const int64_t rows_a = p.M - m0;
    const int64_t rows_b = p.N - n0;
    const int64_t bytes_a = rows_a * K * ES;
    const int64_t bytes_b = rows_b * K * ES;
    const i32x4 rsrc_a = make_rsrc(Ab, (uint32_t)(bytes_a < (int64_t)kOutOfRange ? bytes_a : kOutOfRange));
    const i32x4 rsrc_b = make_rsrc(Bb, (uint32_t)(bytes_b < (int64_t)kOutOfRange ? bytes_b : kOutOfRange));

    // ---- per-lane load offsets: lane -> (row r = lane/8 of the group, physical column lane%8)
    // The logical 16-byte column held at physical column c of row r is c ^ swz(r).
    uint32_t voff_a[A_LOADS], voff_b[B_LOADS];
    int col_a[A_LOADS], col_b[B_LOADS];
    const int64_t row_bytes_g = K * ES;
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int g = wave + j * NW;
        const int r = g * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        col_a[j] = c;
        voff_a[j] = (r < rows_a) ? (uint32_t)(r * row_bytes_g + c * 16) : kOutOfRange;
    }
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int g = wave + j * NW;
        const int r = g * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        col_b[j] = c;
        voff_b[j] = (r < rows_b) ? (uint32_t)(r * row_bytes_g + c * 16) : kOutOfRange;
    }
    const uint32_t smem_base = lds_addr(smem);
    const int64_t k_bytes = K * ES;

    auto issue = [&](int chunk, int slot) {
        const int64_t kb = (int64_t)(chunk0 + chunk) * kRowBytes;   // byte offset of the chunk in a row
        const int64_t rem = k_bytes - kb;                            // bytes of this row left from kb
        const uint32_t soff = (uint32_t)kb;
        const uint32_t sbase = smem_base + slot * SLOT_BYTES;
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j) {
            const int g = wave + j * NW;
            uint32_t v = (col_a[j] * 16 < rem) ? voff_a[j] : kOutOfRange;
            dma16(rsrc_a, sbase + g * 1024, v, soff);
        }
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j) {
            const int g = wave + j * NW;
            uint32_t v = (col_b[j] * 16 < rem) ? voff_b[j] : kOutOfRange;
            dma16(rsrc_b, sbase + BM * kRowBytes + g * 1024, v, soff);
        }
    };

    // ---- operand read offsets (within a slot)
    const int wm = wave % WAVES_M;
    const int wn = wave / WAVES_M;
    const int r16 = lane & 15;
    const int grp = lane >> 4;
    const int sw = swz(r16);
    uint32_t rd_a = (uint32_t)((wm * WTM + r16) * kRowBytes);
    uint32_t rd_b = (uint32_t)(BM * kRowBytes + (wn * WTN + r16) * kRowBytes);

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int slot) {
        const char *base = smem + slot * SLOT_BYTES;
#pragma unroll
        for (int ks = 0; ks < kStepsPerChunk; ++ks) {
            const int col = ((ks * 4 + grp) ^ sw) * 16;
            i32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                fa[i] = *reinterpret_cast<const i32x4 *>(base + rd_a + i * 16 * kRowBytes + col);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                fb[j] = *reinterpret_cast<const i32x4 *>(base + rd_b + j * 16 * kRowBytes + col);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = Elem<T>::mfma_step(fb[j], fa[i], acc[i][j]);
        }
    };

    // ---- the prefetch ring
    if constexpr (P == 0) {
        for (int i = 0; i < nk; ++i) {
            lds_barrier();                 // everyone is done reading the single slot
            issue(i, 0);
            wait_vmcnt<0>();
            lds_barrier();                 // every wave's part of chunk i has landed
            compute(0);
        }
    } else {
#pragma unroll
        for (int i = 0; i < P; ++i)
            if (i < nk) issue(i, i);
        int slot = 0;
        for (int i = 0; i < nk; ++i) {
            // chunks issued after chunk i so far: min(P - 1, nk - 1 - i)
            if (nk - 1 - i >= P - 1)
                wait_vmcnt<LOADS * (P - 1)>();
            else
                wait_vmcnt<0>();
            lds_barrier();                 // chunk i visible to all; slot (i-1) mod SLOTS free
            if (i + P < nk) {
                int ns = slot + P;
                if (ns >= SLOTS) ns -= SLOTS;
                issue(i + P, ns);
            }
            compute(slot);
            slot = (slot + 1 == SLOTS) ? 0 : slot + 1;
        }
    }

    // ---- epilogue: lane owns C[m][n..n+3] for every fragment (i, j)
    const int64_t M = p.M, N = p.N;
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t m = m0 + wm * WTM + i * 16 + r16;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int64_t n = n0 + wn * WTN + j * 16 + grp * 4;
            f32x4 v = acc[i][j];
            if constexpr (MODE == MODE_PARTIAL) {
                float *W = reinterpret_cast<float *>(p.C) + ((int64_t)s * p.L + l) * M * N + m * N;
                if (vec_ok && n + 3 < N) {
                    *reinterpret_cast<f32x4v *>(W + n) = f32x4v{v[0], v[1], v[2], v[3]};
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (n + q < N) W[n + q] = v[q];
                }
            } else {
                T *Cr = reinterpret_cast<T *>(p.C) + ((int64_t)l * M + m) * N;
                const float y0 = apply_epilogue<MODE>(v[0]);
                const float y1 = apply_epilogue<MODE>(v[1]);
                const float y2 = apply_epilogue<MODE>(v[2]);
                const float y3 = apply_epilogue<MODE>(v[3]);
                if (vec_ok && n + 3 < N) {
                    Elem<T>::store4(Cr + n, y0, y1, y2, y3);
                } else {
                    const float y[4] = {y0, y1, y2, y3};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (n + q < N) Cr[n + q] = Elem<T>::from_f32(y[q]);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ split-K reduction

// C = epilogue( sum_{s=0}^{S-1} W[s] ), summed in ascending s.  Four elements a
// thread when every split's slice stays 16-byte aligned (total % 4 == 0),
// else one.
template <class T, int MODE>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ W, T *__restrict__ C,
                                                            int64_t total, int split)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t first = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if ((total & 3) == 0) {
        const int64_t nvec = total >> 2;
        for (int64_t v = first; v < nvec; v += stride) {
            f32x4v sum = *reinterpret_cast<const f32x4v *>(W + v * 4);
            for (int s = 1; s < split; ++s) {
                const f32x4v x = *reinterpret_cast<const f32x4v *>(W + (int64_t)s * total + v * 4);
                sum[0] += x[0];
                sum[1] += x[1];
                sum[2] += x[2];
                sum[3] += x[3];
            }
            Elem<T>::store4(C + v * 4, apply_epilogue<MODE>(sum[0]), apply_epilogue<MODE>(sum[1]),
                            apply_epilogue<MODE>(sum[2]), apply_epilogue<MODE>(sum[3]));
        }
    } else {
        for (int64_t e = first; e < total; e += stride) {
            float sum = W[e];
            for (int s = 1; s < split; ++s)
                sum += W[(int64_t)s * total + e];
            C[e] = Elem<T>::from_f32(apply_epilogue<MODE>(sum));
        }
    }
}

// ------------------------------------------------------------------ general kernel

// Any alignment, any K: element-wise bounds-checked loads into LDS (as fp32),
// 64 x 64 output tile, 256 threads, 4 x 4 outputs a thread, fp32 FMA.
template <class T, int MODE>
__global__ __launch_bounds__(256) void gemm_general_kernel(const T *__restrict__ A, const T *__restrict__ B,
                                                           T *__restrict__ C, int64_t M, int64_t N, int64_t K,
                                                           int32_t tiles_m, int32_t tiles_n)
{
    constexpr int TB = 64, KB = 16;
    __shared__ float sa[KB][TB + 1];
    __shared__ float sb[KB][TB + 1];
    int t = blockIdx.x;
    const int tm = t % tiles_m;
    t /= tiles_m;
    const int tn = t % tiles_n;
    const int l = t / tiles_n;
    const int64_t m0 = (int64_t)tm * TB, n0 = (int64_t)tn * TB;
    const T *Ab = A + (int64_t)l * M * K;
    const T *Bb = B + (int64_t)l * N * K;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < K; k0 += KB) {
        for (int e = threadIdx.x; e < TB * KB; e += 256) {
            const int r = e / KB, kk = e % KB;
            const int64_t ma = m0 + r, nb = n0 + r, k = k0 + kk;
            sa[kk][r] = (ma < M && k < K) ? Elem<T>::to_f32(Ab[ma * K + k]) : 0.0f;
            sb[kk][r] = (nb < N && k < K) ? Elem<T>::to_f32(Bb[nb * K + k]) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = sa[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = sb[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t n = n0 + tx * 4 + j;
            if (n < N) C[((int64_t)l * M + m) * N + n] = Elem<T>::from_f32(apply_epilogue<MODE>(acc[i][j]));
        }
    }
}

}  // namespace gmk
